"""MI355X-native ensemble ODE solves with exact discrete-adjoint gradients.

A trajectory per GPU lane is integrated adaptively (Tsit5, or Rosenbrock23 for
stiff systems) while its accepted step sizes are recorded; the gradient of a
scalar ensemble loss is the reverse-mode derivative of the fixed-step replay of
that record (arXiv 2609.02876, Sec. 2.1 and 3.1).  The work runs in the HIP
library libdao.so behind the C ABI of include/dao.h; this package binds it.
"""
from ._lib import DaoError, dao_version  # noqa: F401  (loads libdao.so or raises)
from .api import (Record, Workspace, cotangent, grad, grad_at, grad_order, sens,  # noqa: F401
                  solve, solve_sens, states_at)

__all__ = ["solve", "solve_sens", "sens", "states_at", "grad", "grad_at", "grad_order",
           "cotangent", "Record", "Workspace", "DaoError", "dao_version"]
