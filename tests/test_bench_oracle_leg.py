"""bench.py calls the oracle only in its CPU-baseline leg.

The leg times the oracle on the host and checks the GPU's results against it; it runs
unless --no-cpu-baseline is given. Every import of the oracle in bench.py must sit inside
the functions that time it or inside an `if oracle_leg(args):` block, so a run without
the leg never executes oracle code. Checked on the source (no GPU needed).
"""
import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LEG_FUNCTIONS = {"_oracle_unit", "cpu_baselines"}


def _imports_oracle(node):
    if isinstance(node, ast.Import):
        return any(a.name == "oracle" or a.name.startswith("oracle.") for a in node.names)
    if isinstance(node, ast.ImportFrom):
        return node.module is not None and (node.module == "oracle" or node.module.startswith("oracle."))
    return False


def _is_leg_test(node):
    return (isinstance(node, ast.If) and isinstance(node.test, ast.Call)
            and isinstance(node.test.func, ast.Name) and node.test.func.id == "oracle_leg")


def _stray_imports(node, inside_leg=False):
    """Line numbers of oracle imports outside the leg."""
    stray = []
    if isinstance(node, ast.FunctionDef) and node.name in LEG_FUNCTIONS:
        inside_leg = True
    if _imports_oracle(node) and not inside_leg:
        stray.append(node.lineno)
    if _is_leg_test(node):
        for child in node.body:
            stray += _stray_imports(child, True)
        for child in node.orelse:
            stray += _stray_imports(child, inside_leg)
        return stray
    for child in ast.iter_child_nodes(node):
        stray += _stray_imports(child, inside_leg)
    return stray


def test_bench_imports_the_oracle_only_in_its_leg():
    with open(os.path.join(ROOT, "bench.py")) as f:
        tree = ast.parse(f.read())
    assert _stray_imports(tree) == []


def test_leg_gate_follows_the_cpu_baseline_flag():
    import argparse
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_src", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    assert bench.oracle_leg(argparse.Namespace(no_cpu_baseline=False))
    assert not bench.oracle_leg(argparse.Namespace(no_cpu_baseline=True))


def test_checker_sees_a_stray_import():
    # the check itself: an oracle import outside the leg is reported, one inside is not
    src = ("def run(args):\n"
           "    import oracle\n"
           "    if oracle_leg(args):\n"
           "        from oracle import vstore\n")
    assert _stray_imports(ast.parse(src)) == [2]
