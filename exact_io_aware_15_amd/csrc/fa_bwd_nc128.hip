// fa_bwd_nc128.hip -- the non-causal d = 128 backward (launch_bwd_nc128).
//
// Same kernels as fa_bwd.hip, instantiated here alone so that this unit keeps
// the compiler's default instruction scheduler: these kernels already use all
// 512 registers per lane, and the ILP-oriented schedule that speeds up the
// other backward kernels makes them spill more (measured 28% slower at
// B=4, H=16, N=2048).
#define FA355_BWD_NC128_UNIT
#include "fa_bwd.hip"
