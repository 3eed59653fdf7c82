// Scaled dot-product attention over one rank's heads (head dim 128, bf16 in
// and out, fp32 softmax and accumulation):
//   ctx = softmax(Q K^T / sqrt(d) + mask) V   per query head, query head h
// reading key/value head h / G (grouped heads), keys t <= the query's
// position when causal.  The queries of sequence b are its last Sq positions
// (position of query s = len_b - Sq + s), so one kernel serves prefill
// (Sq = len) and decode against a cache (Sq small, len up to Lk).
//
// Two kernels, picked by the number of query rows that share one key/value
// head (G * Sq):
//
// * attn_fwd_kernel (many rows: prefill), on the matrix cores.  A workgroup
//   takes 128 queries of one head (4 waves x 32) and walks the key tiles (64
//   keys) through two LDS stages filled by direct global->LDS DMA.  Each
//   wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K the first
//   operand, its Q fragments held in registers for the whole walk), so every
//   lane owns one query: the running max, the running sum and the output
//   rescale are per-lane scalars.  The exponentials P^T are in the layout of
//   the second operand of O^T = V^T P^T, so they go to the matrix cores
//   straight from registers; V^T comes from the row-major V tile through the
//   LDS transpose read (ds_read_b64_tr_b16): in each group of 16 lanes, lane
//   i gets element i%4 of the 8-byte rows addressed by lanes 4j + i/4.
//   The online softmax (running max and sum, output rescale) is the flash
//   attention recurrence (Dao et al., arXiv:2205.14135).
// * attn_decode_kernel (a few rows: decode), memory-bound: the keys of a
//   sequence are split into chunks spread over many workgroups; each streams
//   its chunk of K and then of V once (the V rows of its first pass of
//   64 or 128 keys requested with their K rows), 16 lanes per 256-byte row,
//   and writes an unnormalised partial (max, sum, weighted values).  Each
//   workgroup then counts its arrival for its (sequence, key/value head);
//   the last to arrive merges the chunks of those query rows in chunk order
//   and resets the counter, so the decode step is one launch and no
//   workgroup waits.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "tp_kernels.h"

namespace tpk {
namespace {

#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4v;
typedef __attribute__((address_space(3))) bf16x4v lds_bf16x4v;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kD = 128;           // head dim
constexpr int kBQ = 128;          // queries per workgroup (4 waves x 32)
constexpr int kBK = 64;           // keys per tile
constexpr int kSlots = kBK * kD / 8;  // 16-byte slots per K or V tile (16 KiB)
constexpr int kDecMaxChunk = kAttnDecMaxChunk;
constexpr int kMaxSplit = kAttnMaxSplit;

struct AttnDev {
    const __bf16 *Q, *K, *V;
    __bf16 *O;
    const int32_t *kv_len;        // [Bs] or nullptr (every sequence has Lk keys)
    int64_t ldq, ldk, ldv, ldo;   // row strides, elements
    int Bs, Sq, Lk, nh, nkv, G;
    int causal;
    float scale_log2;             // log2(e) / sqrt(d)
};

__device__ __forceinline__ int seq_len(const AttnDev &a, int b)
{
    const int len = a.kv_len ? a.kv_len[b] : a.Lk;
    return min(max(len, 0), a.Lk);
}

// s_waitcnt immediates (gfx9 encoding): vmcnt = vm, expcnt and lgkmcnt any.
__host__ __device__ constexpr int wait_vm(int vm) { return (vm & 0xF) | (0x7 << 4) | (0xF << 8) | ((vm >> 4) << 14); }
constexpr int kWaitLgkm0 = 0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14);

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- prefill
// LDS tiles: 64 rows (keys) of 256 bytes = 16 chunks of 16 bytes.
//  K: chunk c of row r sits at slot c ^ (r & 15): a fragment read (16
//     consecutive rows, one chunk) hits 16 different slots.
//  V: chunk c of row r sits at slot c ^ 4(r & 3): a transpose read (4
//     consecutive rows x 4 chunks per 32 lanes) hits 16 different slots.
// Causal query tiles differ in cost (tile qt walks about qt+1 key tiles).
// Items are ranked by cost, heaviest first.  When every workgroup is
// resident at once (grid <= resident), workgroup i of the first half takes
// item i and workgroup i of the second half the item of mirrored rank, so
// the two workgroups that share a CU sum to about the same cost; otherwise
// workgroups take items heaviest first as slots free up.
__device__ __forceinline__ int item_of_block(int bid, int grid, int resident)
{
    if (grid > resident) return bid;
    const int half = (grid + 1) / 2;
    return bid < half ? bid : grid - 1 - (bid - half);
}

__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(AttnDev a, int nqt, int resident)
{
    // one array per stage and operand: the compiler then knows which tile
    // a read touches and does not wait for the DMA filling the other stage
    __shared__ u32x4 k0_lds[kSlots];
    __shared__ u32x4 v0_lds[kSlots];
    __shared__ u32x4 k1_lds[kSlots];
    __shared__ u32x4 v1_lds[kSlots];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int per_qt = a.Bs * a.nh;
    const int item = item_of_block((int)blockIdx.x, (int)gridDim.x, resident);
    const int qt = nqt - 1 - item / per_qt;   // items ranked by cost
    const int rem = item % per_qt;
    const int b = rem / a.nh, hq = rem % a.nh, g = hq / a.G;
    const int len = seq_len(a, b);
    const int off = len - a.Sq;                          // position of query s is off + s
    const int q0 = qt * kBQ + wave * 32;                 // this wave's first query
    const int h = lane >> 5, col = lane & 31;

    // keys the workgroup needs, and the last position any of this wave's rows sees
    const int wg_last = min(qt * kBQ + kBQ, a.Sq) - 1;
    const int keys = max(0, a.causal ? min(len, off + wg_last + 1) : len);
    const int ntiles = (keys + kBK - 1) / kBK;
    const bool w_rows = q0 < a.Sq;
    const int w_last_pos = off + min(q0 + 31, a.Sq - 1);

    // Q fragments: lane holds query q0 + col, dims 16t + 8h .. +7 for t = 0..7
    const __bf16 *qb = a.Q + (int64_t)b * a.Sq * a.ldq + hq * kD;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (uint32_t)(((int64_t)a.Sq * a.ldq - hq * kD) * 2));
    bf16x8 qf[8];
    {
        const uint32_t vo = (uint32_t)(((int64_t)(q0 + col) * a.ldq + 8 * h) * 2);
#pragma unroll
        for (int t = 0; t < 8; ++t) qf[t] = __builtin_bit_cast(bf16x8, buf_load16(rq, vo + t * 32, 0));
    }

    // K/V rows past the sequence's length read as zero
    const __bf16 *kb_ = a.K + (int64_t)b * a.Lk * a.ldk + g * kD;
    const __bf16 *vb_ = a.V + (int64_t)b * a.Lk * a.ldv + g * kD;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb_, (uint32_t)max<int64_t>(0, ((int64_t)len * a.ldk - g * kD) * 2));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb_, (uint32_t)max<int64_t>(0, ((int64_t)len * a.ldv - g * kD) * 2));

    // DMA geometry: instruction j of wave w fills the 1 KiB block 4j + w of a
    // tile, rows 16j + 4w + lane/16; lane L lands in slot L%16 and fetches
    // the logical chunk that the swizzle puts there.
    const int drow = 4 * wave + (lane >> 4);
    const int kchunk = (lane & 15) ^ (drow & 15);
    const int vchunk = (lane & 15) ^ (4 * (drow & 3));
    const uint32_t k_vo = (uint32_t)((drow * a.ldk + kchunk * 8) * 2);
    const uint32_t v_vo = (uint32_t)((drow * a.ldv + vchunk * 8) * 2);
    const uint32_t k_jstep = (uint32_t)(16 * a.ldk * 2), v_jstep = (uint32_t)(16 * a.ldv * 2);
    const uint32_t k_tstep = (uint32_t)(kBK * a.ldk * 2), v_tstep = (uint32_t)(kBK * a.ldv * 2);

    auto issue = [&](u32x4 *kst, u32x4 *vst, int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t vo = k_vo + j * k_jstep + kt * k_tstep;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, LDS_PTR(kst + (4 * j + wave) * 64), 16, vo, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t vo = v_vo + j * v_jstep + kt * v_tstep;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, LDS_PTR(vst + (4 * j + wave) * 64), 16, vo, 0, 0, 0);
        }
    };

    // K fragment reads: row kb*32 + col, chunk 2t + h
    const int kfrag = col * 16;
    // V transpose reads: in a group of 16 lanes, lane i addresses row
    // keyoff + (i/4)%4 ... see the header; per lane: row offset rr, the
    // chunk's low bits, the 8-byte half, and the d-block dependent high bits.
    const int rr = (lane >> 2) & 3;
    const int vlow = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int vbyte = (4 * h + rr) * 256 + 16 * vlow + 8 * (lane & 1);

    if (ntiles > 0) issue(k0_lds, v0_lds, 0);

    float m_run = -1e30f, l_run = 0.0f;
    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
    const int my_pos = off + q0 + col;
    // loop-invariant lane offsets: the V transpose reads of each d-block,
    // and the partner lane (the other key half of the same query)
    int vt_off[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) vt_off[db] = vbyte + 64 * (db ^ rr);
    const int half_swap = (lane ^ 32) << 2;

    // One key tile from the stage (kst, vst).  A single barrier per tile:
    // once every wave has passed it, tile kt has landed and no wave still
    // reads the other stage (tile kt-1), which is then refilled with tile
    // kt+1 while this tile is computed.
    auto tile = [&](int kt, u32x4 *kst, u32x4 *vst, u32x4 *kother, u32x4 *vother) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(wait_vm(0) & kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
        if (kt + 1 < ntiles) issue(kother, vother, kt + 1);

        const int k0 = kt * kBK;
        if (w_rows && (!a.causal || k0 <= w_last_pos)) {
            // S^T tile: keys (k0 + 32kb + ...) x this wave's 32 queries
            f32x16 s[2] = {f32x16{}, f32x16{}};
            bf16x8 kf[8][2];
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)   // row kb*32 + col, whose low 4 bits are col's
                    kf[t][kb] = __builtin_bit_cast(bf16x8, kst[kfrag + kb * 512 + ((2 * t + h) ^ (col & 15))]);
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t][kb], qf[t], s[kb], 0, 0, 0);
            // the fragment reads run two k-steps ahead of the MFMAs (left
            // alone, the scheduler issues each pair of reads right before
            // its MFMAs and waits out the LDS latency every time)
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int t = 0; t < 6; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_barrier(0);
            // lane: query q0 + col; element r of s[kb]: key k0 + 32kb + 8(r/4) + 4h + r%4.
            // Only tiles on the diagonal or past the sequence's end need the mask.
            if ((k0 + kBK > len) || (a.causal && k0 + kBK - 1 > off + q0)) {
                const int lim = a.causal ? min(len - 1, my_pos) : len - 1;   // last visible key
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                        s[kb][r] = key > lim ? -INFINITY : s[kb][r];
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(half_swap, __builtin_bit_cast(int, mx)))) *
                 a.scale_log2;
            // Lazy rescale: the reference max m_run (log2 units) only moves
            // when a tile's max exceeds it by more than 8, so the weights stay
            // <= 2^8 and the output is rescaled only on those tiles; the sum
            // and the output share the reference, so the result is the same.
            const bool grow = mx > m_run + 8.0f;
            if (__builtin_amdgcn_ballot_w64(grow)) {
                const float m_new = grow ? mx : m_run;
                const float alpha = fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < 4; ++db) acc[db] *= alpha;
            }
            float ls = 0.0f;
            bf16x8 pb[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(s[kb][r], a.scale_log2, -m_run));
                    ls += p;
                    pb[kb][r >> 3][r & 7] = (__bf16)p;
                }
            l_run += ls;
            // O^T += V^T P^T; k-slot e of lane half h is key 16ks + 8(e/4) + 4h + e%4 of block kb
            const lds_char *vt = reinterpret_cast<const lds_char *>(LDS_PTR(vst));
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int kbase = (kb * 32 + ks * 16) * 256;
#pragma unroll
                    for (int db = 0; db < 4; ++db) {
                        const int o = kbase + vt_off[db];
                        const bf16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4v *)(vt + o));
                        const bf16x4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4v *)(vt + o + 8 * 256));
                        const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kb][ks], acc[db], 0, 0, 0);
                    }
                }
        }
    };
    for (int kt = 0; kt < ntiles; kt += 2) {
        tile(kt, k0_lds, v0_lds, k1_lds, v1_lds);
        if (kt + 1 < ntiles) tile(kt + 1, k1_lds, v1_lds, k0_lds, v0_lds);
    }

    // normalise and store: lane holds query q0 + col, dims 32db + 8(r/4) + 4h + r%4
    const float lt = l_run + __shfl_xor(l_run, 32);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const int q = q0 + col;
    if (q < a.Sq) {
        __bf16 *o = a.O + ((int64_t)b * a.Sq + q) * a.ldo + hq * kD + 4 * h;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const bf16x4 y = {(__bf16)(acc[db][4 * r4] * inv), (__bf16)(acc[db][4 * r4 + 1] * inv),
                                  (__bf16)(acc[db][4 * r4 + 2] * inv), (__bf16)(acc[db][4 * r4 + 3] * inv)};
                *reinterpret_cast<bf16x4 *>(o + 32 * db + 8 * r4) = y;
            }
    }
}

// ---------------------------------------------------------------- decode
// Sum over the 16 lanes of a row (DPP: swap neighbours, swap pairs, mirror
// within 8, mirror within 16); every lane of the row ends with the total.
__device__ __forceinline__ float row16_sum(float x)
{
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    return x;
}

__device__ __forceinline__ void bf16x8_to_f32(u32x4 w, float *f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
        f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
}

// Device-coherent accesses to the split-key partials: relaxed atomics at
// agent scope, which bypass the per-XCD L2s, so a workgroup on another XCD
// reads what was written.
__device__ __forceinline__ void publish(float *p, float x)
{
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fetch(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup (b, g, c): keys [c*chunk, (c+1)*chunk) of sequence b against the
// NR = G*Sq query rows that read key/value head g (row r = gq*Sq + s is query
// s of head g*G + gq).  Lane layout over a K or V row: lanes 16k .. 16k+15
// hold row k of the wave's 4, 16 bytes (8 dims) each; a pass over the chunk
// takes 16*UR keys, UR rows in flight per lane.
// Partial of row r, chunk c: max m, sum l = sum_t 2^(x_t - m), o[d] =
// sum_t 2^(x_t - m) v_t[d], x_t the scaled score in log2 units.
template <int NR, int UR>
__global__ void __launch_bounds__(256) attn_decode_kernel(AttnDev a, int chunk, int nsplit, float *ws_o, float *ws_ml,
                                                          unsigned *arrivals)
{
    // scores then weights [key][row], then per-wave partial outputs; the
    // merge reuses the space for the chunk weights of two rows at a time
    constexpr int kPart = kDecMaxChunk * NR + 4 * NR * kD;
    __shared__ float smem[kPart > 2 * kMaxSplit ? kPart : 2 * kMaxSplit];
    float(*p_lds)[NR] = reinterpret_cast<float(*)[NR]>(smem);
    float(*red)[NR][kD] = reinterpret_cast<float(*)[NR][kD]>(smem + kDecMaxChunk * NR);
    __shared__ float ml[NR][2];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = (int)blockIdx.x % nsplit;
    const int bg = (int)blockIdx.x / nsplit;
    const int b = bg / a.nkv, g = bg % a.nkv;
    const int len = seq_len(a, b);
    const int off = len - a.Sq;
    const int k_begin = c * chunk;
    const int nk = max(0, min(chunk, len - k_begin));
    const int rows = a.G * a.Sq;
    const int kk = lane >> 4, cc = lane & 15;

    // query rows, fp32: lane holds dims 8cc .. 8cc+7 of every row
    float qv[NR][8];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int rr = r < rows ? r : 0;
        const int gq = rr / a.Sq, s = rr % a.Sq;
        const __bf16 *qp = a.Q + ((int64_t)b * a.Sq + s) * a.ldq + (g * a.G + gq) * kD + 8 * cc;
        bf16x8_to_f32(*reinterpret_cast<const u32x4 *>(qp), qv[r]);
    }

    // the chunk's rows of head g; rows past the chunk's valid keys read zero
    const __bf16 *kb_ = a.K + ((int64_t)b * a.Lk + k_begin) * a.ldk + g * kD;
    const __bf16 *vb_ = a.V + ((int64_t)b * a.Lk + k_begin) * a.ldv + g * kD;
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc(kb_, nk > 0 ? (uint32_t)(((int64_t)(nk - 1) * a.ldk + kD) * 2) : 0u);
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(vb_, nk > 0 ? (uint32_t)(((int64_t)(nk - 1) * a.ldv + kD) * 2) : 0u);
    const uint32_t lane_b = 16u * cc;

    // scores: wave w takes keys 16i + 4w + kk, UR rows in flight per lane.
    // The value rows of the first pass's keys do not depend on the scores:
    // they are requested right behind their key rows and stream under the
    // scores and the softmax (one sequence in 64-key chunks: 12.53 -> 11.89
    // us, bitwise equal; 8 and 32 sequences unchanged).
    u32x4 vfirst[UR];
    for (int base = 0; base < nk; base += 16 * UR) {
        u32x4 kr[UR];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int t = base + 16 * u + 4 * wave + kk;
            kr[u] = buf_load16(rk, (uint32_t)(t * a.ldk * 2) + lane_b, 0);
        }
        if (base == 0) {
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int t = 16 * u + 4 * wave + kk;
                vfirst[u] = buf_load16(rv, (uint32_t)(t * a.ldv * 2) + lane_b, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int t = base + 16 * u + 4 * wave + kk;
            float kf[8];
            bf16x8_to_f32(kr[u], kf);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                float dot = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) dot = fmaf(qv[r][e], kf[e], dot);
                dot = row16_sum(dot) * a.scale_log2;
                const int s = r % a.Sq;
                const bool vis = t < nk && !(a.causal && k_begin + t > off + s);
                if (cc == r && t < nk) p_lds[t][r] = vis ? dot : -INFINITY;
            }
        }
    }
    __syncthreads();

    // per row: max and sum over the chunk, scores -> weights
    for (int r = wave; r < NR; r += 4) {
        float mx = -INFINITY;
        for (int t = lane; t < nk; t += 64) mx = fmaxf(mx, p_lds[t][r]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
        const float mref = mx > -INFINITY ? mx : -1e30f;
        float sum = 0.0f;
        for (int t = lane; t < nk; t += 64) {
            const float p = fast_exp2(p_lds[t][r] - mref);
            p_lds[t][r] = p;
            sum += p;
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m);
        if (lane == 0) {
            ml[r][0] = mref;
            ml[r][1] = sum;
        }
    }
    __syncthreads();

    // weighted values
    float o[NR][8];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[r][e] = 0.0f;
    for (int base = 0; base < nk; base += 16 * UR) {
        u32x4 vr[UR];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int t = base + 16 * u + 4 * wave + kk;
            vr[u] = base == 0 ? vfirst[u] : buf_load16(rv, (uint32_t)(t * a.ldv * 2) + lane_b, 0);
        }
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int t = base + 16 * u + 4 * wave + kk;
            if (t < nk) {
                float vf[8];
                bf16x8_to_f32(vr[u], vf);
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const float p = p_lds[t][r];
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[r][e] = fmaf(p, vf[e], o[r][e]);
                }
            }
        }
    }
    // sum the wave's 4 key rows (lanes cc, cc+16, cc+32, cc+48), then the 4 waves
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = o[r][e];
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            if (kk == 0) red[wave][r][8 * cc + e] = x;
        }
    __syncthreads();
    for (int i = threadIdx.x; i < rows * kD; i += 256) {
        const int r = i / kD, d = i % kD;
        const float x = red[0][r][d] + red[1][r][d] + red[2][r][d] + red[3][r][d];
        const int gq = r / a.Sq, s = r % a.Sq;
        const int64_t row = (((int64_t)c * a.Bs + b) * a.Sq + s) * a.nh + g * a.G + gq;
        publish(ws_o + row * kD + d, x);
        if (d == 0) {
            publish(ws_ml + 2 * row, ml[r][0]);
            publish(ws_ml + 2 * row + 1, ml[r][1]);
        }
    }

    // Count the arrival; the last of the nsplit workgroups of (b, g) to
    // arrive merges every chunk of its rows and returns the counter to zero
    // for the next call.  No workgroup waits on another.  The partials are
    // written and read with device-coherent accesses (they bypass the
    // per-XCD L2s), and every store has completed before the arrival is
    // counted, so the merging workgroup reads all of them; no L2 write-back
    // or invalidation is needed (an agent-scope fence here, which does both,
    // took the M = 8 decode step from 20 to 159 us).  The merge sums the
    // chunks in chunk order, so the result does not depend on which
    // workgroup arrives last.
    __shared__ int merge;
    __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores have completed
    __syncthreads();
    if (threadIdx.x == 0)
        merge = __hip_atomic_fetch_add(arrivals + bg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (unsigned)(nsplit - 1);
    __syncthreads();
    if (!merge) return;

    // merge, two query rows at a time, one half-workgroup (128 lanes, one
    // per dim) per row: weight of chunk c = 2^(m_c - M) (chunks without a
    // visible key weigh 0), ctx = sum_c w_c o_c / sum_c w_c l_c
    __shared__ float hred[2][2];
    const int half = threadIdx.x >> 7, t = threadIdx.x & 127, hw = (threadIdx.x >> 6) & 1;
    float *const wts = smem + half * kMaxSplit;
    const int64_t stride = (int64_t)a.Bs * a.Sq * a.nh;
    for (int r0 = 0; r0 < rows; r0 += 2) {
        const int r = r0 + half;
        const bool live = r < rows;
        const int rr = live ? r : 0;
        const int gq = rr / a.Sq, sq = rr % a.Sq;
        const int64_t qrow = ((int64_t)b * a.Sq + sq) * a.nh + g * a.G + gq;
        float M = -INFINITY;
        for (int cc2 = t; cc2 < nsplit; cc2 += kD) {
            const float m2x = fetch(ws_ml + 2 * (cc2 * stride + qrow)), m2y = fetch(ws_ml + 2 * (cc2 * stride + qrow) + 1);
            if (m2y > 0.0f) M = fmaxf(M, m2x);
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m));
        if ((t & 63) == 0) hred[half][hw] = M;
        __syncthreads();
        M = fmaxf(hred[half][0], hred[half][1]);
        __syncthreads();
        float L = 0.0f;
        for (int cc2 = t; cc2 < nsplit; cc2 += kD) {
            const float m2x = fetch(ws_ml + 2 * (cc2 * stride + qrow)), m2y = fetch(ws_ml + 2 * (cc2 * stride + qrow) + 1);
            const float w = m2y > 0.0f ? fast_exp2(m2x - M) : 0.0f;
            wts[cc2] = w;
            L = fmaf(m2y, w, L);
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) L += __shfl_xor(L, m);
        if ((t & 63) == 0) hred[half][hw] = L;
        __syncthreads();
        L = hred[half][0] + hred[half][1];
        float O = 0.0f;
        int k = 0;
        for (; k + 8 <= nsplit; k += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = fetch(ws_o + ((k + u) * stride + qrow) * kD + t);
#pragma unroll
            for (int u = 0; u < 8; ++u) O = fmaf(v[u], wts[k + u], O);
        }
        for (; k < nsplit; ++k) O = fmaf(fetch(ws_o + (k * stride + qrow) * kD + t), wts[k], O);
        if (live) {
            const int64_t bs = qrow / a.nh;
            const int hq = (int)(qrow % a.nh);
            a.O[bs * a.ldo + hq * kD + t] = (__bf16)(L > 0.0f ? O / L : 0.0f);
        }
        __syncthreads();   // wts and hred are reused by the next pair of rows
    }
    if (threadIdx.x == 0) __hip_atomic_store(arrivals + bg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int NR>
hipError_t launch_decode(const AttnDev &d, int chunk, int nsplit, float *ws_o, float *ws_ml, unsigned *arrivals,
                         hipStream_t s)
{
    const int grid = d.Bs * d.nkv * nsplit;
    // A chunk of at most 128 keys goes in one pass of 8 key rows per lane
    // (its values requested with it); longer chunks in passes of 4.  One
    // sequence (16 chunks of 128): 11.47 -> 10.29 us, 8 sequences 21.02 ->
    // 20.55 us; 32 sequences (chunks of 512) took 57.0 against 53.9 us with 8
    // rows.  Bitwise equal: a lane visits the same keys in the same order.
    if (chunk <= 128)
        hipLaunchKernelGGL((attn_decode_kernel<NR, 8>), dim3(grid), dim3(256), 0, s, d, chunk, nsplit, ws_o, ws_ml,
                           arrivals);
    else
        hipLaunchKernelGGL((attn_decode_kernel<NR, 4>), dim3(grid), dim3(256), 0, s, d, chunk, nsplit, ws_o, ws_ml,
                       arrivals);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs &x, int num_cu, hipStream_t s)
{
    AttnDev d{};
    d.Q = static_cast<const __bf16 *>(x.Q);
    d.K = static_cast<const __bf16 *>(x.K);
    d.V = static_cast<const __bf16 *>(x.V);
    d.O = static_cast<__bf16 *>(x.O);
    d.kv_len = x.kv_len;
    d.ldq = x.ldq;
    d.ldk = x.ldk;
    d.ldv = x.ldv;
    d.ldo = x.ldo;
    d.Bs = (int)x.Bs;
    d.Sq = (int)x.Sq;
    d.Lk = (int)x.Lk;
    d.nh = x.nh;
    d.nkv = x.nkv;
    d.G = x.nh / x.nkv;
    d.causal = x.causal ? 1 : 0;
    d.scale_log2 = (float)(1.4426950408889634 / 11.313708498984761);   // log2(e) / sqrt(128)
    const AttnPlan p = attn_plan(x.Bs, x.Sq, x.Lk, x.nh, x.nkv);
    if (!p.decode) {
        const int nqt = (int)((x.Sq + kBQ - 1) / kBQ);
        const int64_t grid = (int64_t)nqt * x.Bs * x.nh;
        // two workgroups per CU (64 KiB of LDS and <= 256 VGPRs each)
        hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)grid), dim3(256), 0, s, d, nqt, 2 * num_cu);
        return hipGetLastError();
    }
    unsigned *arrivals = static_cast<unsigned *>(x.ws);
    float *ws_o = reinterpret_cast<float *>(static_cast<char *>(x.ws) + p.partials_offset);
    float *ws_ml = ws_o + (size_t)p.nsplit * x.Bs * x.Sq * x.nh * kD;
    const int rows = d.G * d.Sq;
    if (rows <= 1) return launch_decode<1>(d, p.chunk, p.nsplit, ws_o, ws_ml, arrivals, s);
    if (rows <= 2) return launch_decode<2>(d, p.chunk, p.nsplit, ws_o, ws_ml, arrivals, s);
    if (rows <= 4) return launch_decode<4>(d, p.chunk, p.nsplit, ws_o, ws_ml, arrivals, s);
    return launch_decode<8>(d, p.chunk, p.nsplit, ws_o, ws_ml, arrivals, s);
}

}  // namespace tpk
