// The op that produces X for the producer-fused int8 linear (internal to
// libw8mp): its kind and parameters, shared by the host launchers and the
// kernels. The device arithmetic is in produce.h.
#pragma once

namespace w8 {

enum : int { kProdNone = 0, kProdRms = 1, kProdGelu = 2 };

struct ProdArgs {
  const float* gamma;   // [K] or null (1)
  const float* scale;   // [K] or null (0)
  const float* shift;   // [K] or null (no addition)
  float eps;
  float* rstd;          // [M]: written by the row pass, read by the fix-up (RMSNorm)
};

}  // namespace w8
