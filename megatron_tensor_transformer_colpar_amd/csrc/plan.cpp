// Host-side launch planning shared by the C ABI's validation and the
// kernels' launchers: which attention kernel a shape takes and how much
// workspace its split-key partials need.  Plain C++ with no device code, so
// the ABI can also be built and checked on a machine without a GPU.
#include <algorithm>
#include <cstdint>

#include "tp_kernels.h"

namespace tpk {

AttnPlan attn_plan(int64_t Bs, int64_t Sq, int64_t Lk, int nh, int nkv)
{
    AttnPlan p{};
    const int64_t rows = (int64_t)(nh / nkv) * Sq;
    // the split-key kernel needs one arrival counter per (sequence, key/value
    // head) in the counter region; more pairs take the matrix-core kernel
    p.decode = rows <= kAttnDecRows && Bs * nkv <= kAttnMaxArrivals;
    if (!p.decode) return p;
    // enough workgroups to cover the chip four times over (a workgroup
    // keeps only 16 KiB of its chunk in flight), at most kAttnDecMaxChunk keys
    // each; measured against two times over: 19.8 vs 22.5 us for 8
    // sequences of 2048 cached keys, 1 and 32 sequences unchanged.  At least
    // 128 keys per chunk: one sequence of 2048 keys in 16 chunks took 11.43
    // us against 11.83 in 32 chunks of 64 and 13.92 in 8 of 256 (the merge
    // reads every chunk's partial after the last arrival)
    const int64_t heads = Bs * nkv;
    int64_t nsplit = heads > 0 ? (1024 + heads - 1) / heads : 1;
    nsplit = std::min<int64_t>(nsplit, (Lk + 127) / 128);
    nsplit = std::max<int64_t>(nsplit, (Lk + kAttnDecMaxChunk - 1) / kAttnDecMaxChunk);
    int64_t chunk = (Lk + nsplit - 1) / nsplit;
    chunk = (chunk + 63) / 64 * 64;
    nsplit = (Lk + chunk - 1) / chunk;
    if (nsplit > kAttnMaxSplit) {   // caches beyond 2M keys take the matrix-core kernel
        p.decode = false;
        return p;
    }
    p.nsplit = (int)nsplit;
    p.chunk = (int)chunk;
    // the arrival counters first, in a region of fixed size (so that no
    // call's partials ever cover another call's counters), then the chunks'
    // partials (weighted values, then max and sum per row)
    const int64_t qrows = Bs * Sq * nh;
    p.partials_offset = (size_t)kAttnMaxArrivals * 4;
    p.ws_bytes = p.partials_offset + (size_t)(nsplit * qrows * (kAttnD + 2) * 4);
    return p;
}

}  // namespace tpk
