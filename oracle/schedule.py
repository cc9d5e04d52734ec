"""Per-layer keep budgets: the pyramid schedules of the pages (oracle).

THIS IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT (see oracle/__init__.py).

Layer l of n keeps the fraction ratio_l of a base budget:

* linear, "KV Cache optimization techniques" tutorial, section 2.3 (the
  PyramidKV manager's default schedule): ratio_l = 1.0 - 0.8 * (l / n);
* quadratic, eviction-and-reuse survey, section 4 (the eviction engine's
  pyramid ratio): ratio_l = r + (1 - r) * (l / n) ** 2. The page sets n = 80
  as an assumption; here n is the layer count given.

The budget is int(base * ratio_l), as the tutorial takes int() of the scaled
length, raised to min_budget. Python floats are IEEE doubles, the arithmetic
the pages' code does.
"""

LINEAR, QUADRATIC = 0, 1


def layer_budgets(schedule: int, num_layers: int, base: int, base_ratio: float = 0.0,
                  min_budget: int = 0) -> list:
    if num_layers < 1 or base < 1 or min_budget < 0:
        raise ValueError("need num_layers >= 1, base >= 1, min_budget >= 0")
    out = []
    for layer in range(num_layers):
        if schedule == LINEAR:
            ratio = 1.0 - 0.8 * (layer / num_layers)
        elif schedule == QUADRATIC:
            if not 0.0 <= base_ratio <= 1.0:
                raise ValueError("base_ratio must lie in [0, 1]")
            ratio = base_ratio + (1 - base_ratio) * (layer / num_layers) ** 2
        else:
            raise ValueError("unknown schedule")
        out.append(max(min_budget, int(base * ratio)))
    return out
