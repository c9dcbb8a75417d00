// Where a kernel takes dt and A from (host and device code share it).
#pragma once
#include <stdint.h>

// With `bias` null, dt and A are used as given (dt > 0, A < 0). With `bias`
// set (the packed-projection entry points), dt holds the projection's raw
// values and A holds A_log: the step before the scan is applied in the
// kernels, dt = softplus(raw + bias[h]) and A = -exp(A_log[h]).
// dts: token stride of dt in elements.
struct DtA {
  int64_t dts;
  const float* bias;
};
