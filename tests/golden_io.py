"""Reader for the hand-worked fixtures under tests/golden/.

Values are exact expressions (numbers, + - * / **, unary minus, sqrt) that
were derived by hand; they are evaluated here with a tiny AST walker so that
no fixture can run code.
"""
import ast
import math
import os
import operator

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_BIN = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv, ast.Pow: operator.pow}


def _eval(node):
    if isinstance(node, ast.Expression):
        return _eval(node.body)
    if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
        return float(node.value)
    if isinstance(node, ast.BinOp) and type(node.op) in _BIN:
        return _BIN[type(node.op)](_eval(node.left), _eval(node.right))
    if isinstance(node, ast.UnaryOp) and isinstance(node.op, (ast.USub, ast.UAdd)):
        x = _eval(node.operand)
        return -x if isinstance(node.op, ast.USub) else x
    if (isinstance(node, ast.Call) and isinstance(node.func, ast.Name)
            and node.func.id == "sqrt" and len(node.args) == 1):
        return math.sqrt(_eval(node.args[0]))
    raise ValueError(f"unsupported fixture expression: {ast.dump(node)}")


def _split_top(text):
    parts, depth, cur = [], 0, []
    for ch in text:
        if ch == "(":
            depth += 1
        elif ch == ")":
            depth -= 1
        if ch == "," and depth == 0:
            parts.append("".join(cur))
            cur = []
        else:
            cur.append(ch)
    parts.append("".join(cur))
    return [p.strip() for p in parts if p.strip()]


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition("=")
            vals = [_eval(ast.parse(p, mode="eval")) for p in _split_top(val)]
            out[key.strip()] = vals if len(vals) != 1 else vals[0]
    return out
