// pkm_update.hpp -- launchers of the value-table update and the slot-usage
// counter (internal to libpkm.so; the public interface is include/pkm.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkm {

struct UpdateParams {
    float lr;
    float b1, b2, eps;      // Adam only
    float c1, c2;           // Adam bias corrections 1 - b1^t, 1 - b2^t
};

// Rows f with slot_start[f + 1] > slot_start[f]: SGD (adam = false) or Adam
// with per-row moments m1, m2 [slots][d_v] (adam = true).  d_v % 8 == 0.
hipError_t launch_sparse_update(int dtype, void *values, const float *dvalues,
                                const int32_t *slot_start, float *m1, float *m2, int64_t slots,
                                int d_v, bool adam, const UpdateParams &prm, hipStream_t stream);

// counts[f] += slot_start[f + 1] - slot_start[f]; *used (if not NULL) = the
// number of f with counts[f] != 0 afterwards.
hipError_t launch_slot_usage(const int32_t *slot_start, int64_t *counts, int64_t slots,
                             int64_t *used, hipStream_t stream);

}  // namespace pkm
