"""Reader for the hand-derived fixtures in tests/golden/ (restricted arithmetic only)."""
import ast
import math
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_NAMES = {"E1": math.exp(-1.0), "E2": math.exp(-2.0)}
_FUNCS = {"exp": math.exp}


def _eval(expr: str) -> float:
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return float(node.value)
        if isinstance(node, ast.Name) and node.id in _NAMES:
            return _NAMES[node.id]
        if isinstance(node, ast.UnaryOp) and isinstance(node.op, (ast.USub, ast.UAdd)):
            v = ev(node.operand)
            return -v if isinstance(node.op, ast.USub) else v
        if isinstance(node, ast.BinOp) and isinstance(node.op, (ast.Add, ast.Sub, ast.Mult, ast.Div)):
            a, b = ev(node.left), ev(node.right)
            return {ast.Add: a + b, ast.Sub: a - b, ast.Mult: a * b, ast.Div: a / b}[type(node.op)]
        if (isinstance(node, ast.Call) and isinstance(node.func, ast.Name) and node.func.id in _FUNCS
                and len(node.args) == 1):
            return _FUNCS[node.func.id](ev(node.args[0]))
        raise ValueError(f"unsupported expression: {ast.dump(node)}")
    return ev(ast.parse(expr.strip(), mode="eval"))


def load_cases(name="hand_rows.txt"):
    cases, cur = [], None
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (x.strip() for x in line.split(":", 1))
            if key == "case":
                cur = {"case": val}
                cases.append(cur)
            elif key in ("calib", "tail_policy", "recon"):
                cur[key] = val
            else:
                vals = [_eval(v) for v in val.split(",")]
                cur[key] = vals if len(vals) > 1 or key in ("s", "u", "r", "t", "ell", "wL", "wN", "wC", "tail") else vals[0]
    return cases
