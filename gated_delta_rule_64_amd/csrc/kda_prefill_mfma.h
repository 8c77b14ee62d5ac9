// Matrix-core (MFMA) chunked prefill for dk = dv = 128 with bf16 inputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda_internal.h"
#include "kda_prefill_common.h"

namespace kda {

bool mfma_prefill_supports(int dk, int dv, DT x);
// Whether the matrix-core kernels derive each chunk slot from cu_seqlens
// themselves (then no chunk map is built before them): up to 64 sequences,
// no snapshots.
bool mfma_inline_map(int N, const Snapshots& snap);
size_t mfma_record_bytes();
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s, int32_t* base, const SlotInfo* slot_info,
                               char* recs);
hipError_t launch_layer_mfma(const LayerArgs& a, hipStream_t s, int32_t* base, const SlotInfo* slot_info,
                             char* recs);

}  // namespace kda
