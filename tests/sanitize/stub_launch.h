// Recorded calls of the host stand-ins for the kernel launchers (stub_launch.cpp).
#pragma once

#include <stdint.h>

#include <vector>

#include "../../packed_int4_convrot_amd/csrc/launch.h"

namespace stub {

enum class Kernel { kNone, kRotateQuant, kAwqGemm, kQuantizeWeights, kGemv, kGemvFused, kSkinnyFused, kSkinny, kGemm, kW4a16Gemv };

struct Call {
    Kernel kernel = Kernel::kNone;
    int64_t M = 0, K = 0, N = 0;
    int G = 0, qmax = 0;
    int64_t ldq = 0;
    bool packed4 = false, tiled = false, a4 = false, per_group = false;
    float x_scale = 0.f;
    const void *x = nullptr, *codes = nullptr, *row_scales = nullptr, *xr = nullptr;
    const void *out = nullptr, *acc = nullptr, *stream = nullptr;
};

extern Call last;         // the most recent launch
extern int next_status;   // returned by the next launch (then reset to 0)
extern int calls;         // launches since reset()
extern std::vector<Call> log;

void reset();
const void *scratch_base();  // host copy of the library scratch (after first use)

}  // namespace stub
