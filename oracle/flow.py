"""Flow-matching Euler update of the latent (float64 oracle).

Pages cited:
  NOTES = papernotes.org, "Live Avatar: Streaming Real-time Audio-Driven Avatar
          Generation with Infinite Length", 损失函数 / 训练策略 (the flow-matching
          loss regresses v_theta(x_t, t, c) onto x_1 - x_0)
  BLOG  = gitcode.csdn.net, "Live Avatar 深度解析：首个 14B 参数实时流式无限时长数字人",
          疑问 6 (four fixed steps t4->t3->t2->t1->t0, one per pipeline GPU) and
          疑问 7 (flow matching predicts the velocity field v)

Reading taken: the linear path x_t = (1 - t) x_0 + t x_1 with x_1 the noise at
t = 1 and x_0 the data at t = 0, so dx_t/dt = x_1 - x_0 = v; the sampler step
from t_i to t_{i-1} is one Euler step x_{t_{i-1}} = x_{t_i} + (t_{i-1} - t_i) v
on the uniform 4-step grid t = 1, 0.75, 0.5, 0.25, 0 (dt = -0.25).  The real
distilled schedule is not printed on the pages (parity unpinned for it).
"""

from __future__ import annotations

import numpy as np


def uniform_grid(steps: int = 4):
    """Timesteps t_steps..t_0 = 1, 1 - 1/steps, ..., 0 (descending)."""
    return [1.0 - i / steps for i in range(steps + 1)]


def euler_step(x: np.ndarray, v: np.ndarray, dt: float) -> np.ndarray:
    """x + dt * v in float64."""
    return np.asarray(x, dtype=np.float64) + float(dt) * np.asarray(v, dtype=np.float64)


def linear_path_point(x0: np.ndarray, x1: np.ndarray, t: float) -> np.ndarray:
    """x_t = (1 - t) x_0 + t x_1 on the flow-matching path (float64)."""
    return (1.0 - t) * np.asarray(x0, dtype=np.float64) + t * np.asarray(x1, dtype=np.float64)
