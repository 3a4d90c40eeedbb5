// decode.hip -- attention of one new token per sequence over its KV cache, SWA and GA.
//
// Operation (Hugging Face Transformers model doc "MiMo-V2-Flash"): with
// past_key_values only the unprocessed token is passed and earlier keys come
// from the cache (MiMoV2FlashModel.forward); SWA layers see keys p-128..p
// (sliding_window 129), GA layers all keys 0..p; a learnable attention sink
// joins each softmax denominator (Key features); 64 query heads share 4 KV
// heads, head_dim 192 for q/k and 128 for v (MiMoV2FlashConfig).
//
// Shared building block: one wave attends the 16 query heads of one KV group
// (GQA packing into the MFMA N dimension) over 32-key tiles with
// v_mfma_f32_16x16x32_bf16.  Loads go through buffer descriptors whose record
// count ends at the last cached key of the sequence: rows past it read as
// zero, so there are no per-key branches, and a tile's position is a scalar
// offset.  K rows are loaded straight into MFMA A-operand registers; V rows are
// loaded into registers, written to a wave-private LDS tile (row-major, the
// 16-byte chunks of row r XOR-swizzled by 2*(r%8) so the transposed reads are
// bank-conflict free) and read back transposed with ds_read_b64_tr_b16.  Two
// tiles are in flight per wave: the next tile's loads are issued before the
// current one is computed.
//
// SWA decode (one workgroup per (sequence, KV group)): the ring slots are
// split into 32-key tiles over the 4 waves, and the waves' partial (m, l, O)
// are merged in LDS together with the sink and the new token, whose score the
// merge threads form as a dot product.
//
// GA decode: split-K.  Workgroup (split s, sequence b) covers keys
// [s*C, (s+1)*C) of the sequence with one wave per KV group, streaming pool
// rows (384 B of K and 256 B of V per group) and writing an unnormalised
// partial (m, l, O) without the sink; the split holding position p adds the
// new token as its last tile.  A second kernel merges the splits of each
// (sequence, head), adds the sink exactly once, and writes O and LSE.
//
// Paged GA pool: pages of P >= 16 rows (a power of two), so each 16-key half
// of a tile lies in one page and gets a descriptor of its own.  The split's
// page numbers (at most 128) are loaded once per wave into two registers and
// picked out per half-tile with a lane read, so the streaming loop issues no
// dependent table loads; tiles, their order and the arithmetic are those of
// the contiguous pool.
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

// Device memory of the no-allocation decode entry point (GA workspace: plan
// header and partial results).  Each GPU the library runs on holds its own
// copy until the process ends.  Host code must not use this name as an
// address: it is a host-side stand-in; noalloc_scratch() returns the device's
// own address of it, looked up once per device.
static __device__ __attribute__((aligned(256))) unsigned char scratch[mimo::kNoAllocScratchBytes];

namespace mimo {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}
namespace {

constexpr int kDqk = 192;
constexpr int kDv = 128;
constexpr int kGroup = 16;
constexpr int kTile = 32;                         // keys per wave tile
constexpr int kVTileBytes = kTile * kDv * 2;      // 8 KB: 32 rows of 256 B
constexpr int kBlockLdsBytes = 4 * kVTileBytes;   // one V tile per wave
// SWA decode's cross-wave merge, in the same LDS once the tiles are done: per
// wave 16 heads x 128 fp32 outputs in rows padded to 132 floats (a row pitch
// of 528 bytes puts the 16 heads' 16-byte writes on distinct banks), then 16
// (m, l) pairs per wave.
constexpr int kMergeRow = kDv + 4;
constexpr int kMergeBytes = (4 * kGroup * kMergeRow + 4 * kGroup * 2) * 4;
constexpr int kSwaLdsBytes = kMergeBytes > kBlockLdsBytes ? kMergeBytes : kBlockLdsBytes;
#ifndef MIMO_GA_DECODE_DEPTH
#define MIMO_GA_DECODE_DEPTH 2
#endif
constexpr int kGaDepth = MIMO_GA_DECODE_DEPTH;    // GA split: tiles in flight beyond the current one
#ifndef MIMO_GA_FP8_DEPTH
#define MIMO_GA_FP8_DEPTH 3
#endif
constexpr int kFp8Depth = MIMO_GA_FP8_DEPTH;      // FP8 split: a tile is half the bytes, so more in flight
constexpr int kSwaDepth = 1;                      // SWA: a wave owns at most a few tiles

// One 32-key tile of a wave: where its K and V rows come from.
struct TileSrc {
    rsrc_t k, v;     // descriptors; bytes past their record count read as zero
    int koff, voff;  // byte offset of the tile's first key row (wave-uniform)
    int nvalid;      // keys [0, nvalid) of the tile are in the key set
};

// A tile of a paged pool: keys 0..15 and 16..31 through descriptors of their
// own (each half lies inside one page), all offsets zero.
struct PagedTileSrc {
    rsrc_t k[2], v[2];
    int nvalid;
};

// Per-wave running state for 16 heads.  Lane l owns head (l % 16); o[db][r]
// is O^T[dv = 16*db + 4*(l/16) + r][head]; m is the same in the 4 lanes of a
// head, l is a per-lane partial sum (the 4 partials add up at the end).
struct WaveAcc {
    f32x4 o[kDv / 16];
    float m, l;
};

// Lane-constant byte offsets inside a tile.  K: lane l supplies MFMA A rows
// key = l%16 (+16 for the second block), d = 8*(l/16) .. +7 of each 32-wide
// K-step (the K-step adds 64 bytes).  V: load i takes key 4i + l/16, 16-byte
// chunk l%16 of that row.
struct LaneOffsets {
    int k0, k1, v;
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane, int g, int rowk, int rowv) {
    const int G = lane >> 4;
    LaneOffsets o;
    o.k0 = (lane & 15) * rowk + g * (kDqk * 2) + G * 16;
    o.k1 = o.k0 + 16 * rowk;
    o.v = G * rowv + g * (kDv * 2) + (lane & 15) * 16;
    return o;
}

__device__ __forceinline__ void issue_k(const TileSrc& t, const LaneOffsets& lo, u32x4 (&k)[12]) {
#pragma unroll
    for (int st = 0; st < kDqk / 32; ++st) {
        k[st] = __builtin_amdgcn_raw_buffer_load_b128(t.k, lo.k0 + 64 * st, t.koff, 0);
        k[6 + st] = __builtin_amdgcn_raw_buffer_load_b128(t.k, lo.k1 + 64 * st, t.koff, 0);
    }
}

__device__ __forceinline__ void issue_v(const TileSrc& t, const LaneOffsets& lo, int rowv, u32x4 (&v)[kTile / 4]) {
#pragma unroll
    for (int i = 0; i < kTile / 4; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(t.v, lo.v, t.voff + 4 * i * rowv, 0);
}

// Paged halves: rows l%16 of each half for K; V load i takes key 4i + l/16,
// i.e. half i/4 at row 4(i%4) + l/16.
__device__ __forceinline__ void issue_k(const PagedTileSrc& t, const LaneOffsets& lo, u32x4 (&k)[12]) {
#pragma unroll
    for (int st = 0; st < kDqk / 32; ++st) {
        k[st] = __builtin_amdgcn_raw_buffer_load_b128(t.k[0], lo.k0 + 64 * st, 0, 0);
        k[6 + st] = __builtin_amdgcn_raw_buffer_load_b128(t.k[1], lo.k0 + 64 * st, 0, 0);
    }
}

__device__ __forceinline__ void issue_v(const PagedTileSrc& t, const LaneOffsets& lo, int rowv,
                                        u32x4 (&v)[kTile / 4]) {
#pragma unroll
    for (int i = 0; i < kTile / 4; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(t.v[i / 4], lo.v, 4 * (i % 4) * rowv, 0);
}

// V rows to the wave's LDS tile: row r = 4i + G, logical chunk lane%16 stored
// at chunk position (lane%16) ^ 2(r%8).  The previous tile's transposed reads were
// issued earlier by this wave, and a wave's LDS operations run in order.
__device__ __forceinline__ void stage_v(const u32x4 (&v)[kTile / 4], char* vbuf, int lane) {
    const int G = lane >> 4;
#pragma unroll
    for (int i = 0; i < kTile / 4; ++i)
        *reinterpret_cast<u32x4*>(vbuf + (4 * i + G) * (kDv * 2) + (((lane & 15) ^ (2 * (4 * (i & 1) + G))) * 16)) = v[i];
    wave_lds_fence();
}

// As stage_v, with rows r >= nvalid stored as zeros: for tiles whose loads
// were issued before the number of valid keys was known (the rows past it may
// hold anything, and a zero probability times a non-finite value is NaN).
__device__ __forceinline__ void stage_v_masked(const u32x4 (&v)[kTile / 4], char* vbuf, int lane, int nvalid) {
    const int G = lane >> 4;
#pragma unroll
    for (int i = 0; i < kTile / 4; ++i) {
        const u32x4 x = (4 * i + G < nvalid) ? v[i] : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(vbuf + (4 * i + G) * (kDv * 2) + (((lane & 15) ^ (2 * (4 * (i & 1) + G))) * 16)) = x;
    }
    wave_lds_fence();
}

// One tile whose K rows are in `k` and whose V rows are staged in `vbuf`.
__device__ __forceinline__ void attend_tile(WaveAcc& acc, const bf16x8 (&qf)[kDqk / 32], const u32x4 (&k)[12],
                                            const char* vbuf, int nvalid, float c_log2, int lane) {
    const int G = lane >> 4;
    f32x4 s[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int st = 0; st < kDqk / 32; ++st) {
        s[0] = mfma_16x16x32(__builtin_bit_cast(bf16x8, k[st]), qf[st], s[0]);
        s[1] = mfma_16x16x32(__builtin_bit_cast(bf16x8, k[6 + st]), qf[st], s[1]);
    }
    // Key of s[blk][r] inside the tile: 16*blk + 4*G + r.
    float mx = -__builtin_inff();
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = (16 * blk + 4 * G + r < nvalid) ? s[blk][r] : -__builtin_inff();
            s[blk][r] = x;
            mx = fmaxf(mx, x);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(acc.m, mx * c_log2);
    const float alpha = fast_exp2(acc.m - m_new);
    float rs = 0.0f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(__builtin_fmaf(s[blk][r], c_log2, -m_new));
            s[blk][r] = p;
            rs += p;
        }
    acc.l = acc.l * alpha + rs;
    acc.m = m_new;
    // P^T as the B operand: position 8*G + t holds key 4*G + t (t < 4) or 16 + 4*G + t - 4.
    const bf16x8 pf = pack_bf16x8(s[0][0], s[0][1], s[0][2], s[0][3], s[1][0], s[1][1], s[1][2], s[1][3]);
    // V^T as the A operand, transposed out of the swizzled row-major tile: this
    // lane addresses row r = 4*G + t' (t' = (lane%16)/4), columns 16*db +
    // 4*(lane%4), i.e. the 32-byte pair db ^ (r%8) (and row r + 16, same pair).
    const int tq = (lane & 15) >> 2;
    const int rsw = 4 * (G & 1) + tq;
    const char* vrow = vbuf + (4 * G + tq) * (kDv * 2) + 8 * (lane & 3);
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) {
        const char* p = vrow + 32 * (db ^ rsw);
        const bf16x8 a = join_tr(lds_read_tr16(reinterpret_cast<const uint16_t*>(p)),
                                 lds_read_tr16(reinterpret_cast<const uint16_t*>(p + 16 * kDv * 2)));
        acc.o[db] = mfma_16x16x32(a, pf, acc.o[db] * alpha);
    }
    wave_lds_fence();  // the next tile's V writes come after these reads
}

// Hooks of the tile loops (used by the fused RoPE): prep() runs once, after
// the first tiles' loads are issued and before any tile is computed (it may
// rewrite qf); khook(i, k) runs on tile i's K registers right before tile i
// is computed.  The defaults do nothing.
struct NoPrep {
    __device__ void operator()() const {}
};
struct NoKHook {
    __device__ void operator()(int, u32x4 (&)[12]) const {}
};

// Runs tiles 0..ntiles-1 (get(i) describes tile i) with the loads of the next
// D tiles in flight: D + 1 register sets rotate, and tile i+D is issued right
// before tile i is staged and computed.  Every step issues its loads
// unconditionally: past the last tile, get() returns an empty tile (a
// descriptor with no records, so the loads return zeros without touching
// memory, and no valid key, so the attention update is an exact no-op).  The
// count of loads in flight is then the same on every path, which keeps the
// compiler's vmcnt bookkeeping exact.
template <int D, class GetTile, class Prep = NoPrep, class KHook = NoKHook>
__device__ __forceinline__ void run_tiles(WaveAcc& acc, const bf16x8 (&qf)[kDqk / 32], char* vbuf, int ntiles,
                                          const GetTile& get, const LaneOffsets& lo, int rowv, float c_log2,
                                          int lane, const Prep& prep = Prep{}, const KHook& khook = KHook{}) {
    if (ntiles <= 0) {
        prep();
        return;
    }
    u32x4 kr[D + 1][12], vr[D + 1][kTile / 4];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const auto t = get(j);
        issue_k(t, lo, kr[j]);
        issue_v(t, lo, rowv, vr[j]);
    }
    prep();
    for (int i0 = 0; i0 < ntiles; i0 += D + 1) {
#pragma unroll
        for (int j = 0; j <= D; ++j) {
            const auto t = get(i0 + j + D);
            issue_k(t, lo, kr[(j + D) % (D + 1)]);
            issue_v(t, lo, rowv, vr[(j + D) % (D + 1)]);
            stage_v(vr[j], vbuf, lane);
            khook(i0 + j, kr[j]);
            attend_tile(acc, qf, kr[j], vbuf, get(i0 + j).nvalid, c_log2, lane);
        }
    }
}

// At most two tiles (a wave's share of a ring of up to 256 slots): both
// tiles' loads are issued up front, unconditionally (tile 1 may be empty), and
// only the second tile's compute depends on ntiles.  V
// rows at or past a tile's nvalid are staged as zeros, so its descriptors may
// cover rows that hold no key yet.
template <class GetTile, class Prep = NoPrep, class KHook = NoKHook>
__device__ __forceinline__ void run_two_tiles(WaveAcc& acc, const bf16x8 (&qf)[kDqk / 32], char* vbuf, int ntiles,
                                              const GetTile& get, const LaneOffsets& lo, int rowv, float c_log2,
                                              int lane, const Prep& prep = Prep{}, const KHook& khook = KHook{}) {
    u32x4 ka[12], kb[12], v[kTile / 4];
    const TileSrc t0 = get(0), t1 = get(1);
    issue_k(t0, lo, ka);
    issue_v(t0, lo, rowv, v);
    issue_k(t1, lo, kb);
    prep();
    stage_v_masked(v, vbuf, lane, t0.nvalid);
    issue_v(t1, lo, rowv, v);  // tile 1's V reuses the registers tile 0's V was staged from
    khook(0, ka);
    attend_tile(acc, qf, ka, vbuf, ntiles > 0 ? t0.nvalid : 0, c_log2, lane);
    if (ntiles > 1) {
        stage_v_masked(v, vbuf, lane, t1.nvalid);
        khook(1, kb);
        attend_tile(acc, qf, kb, vbuf, t1.nvalid, c_log2, lane);
    }
}

// Q^T fragments of the 16 heads of group g for batch row b: lane holds
// q[b][16*g + lane%16][32*st + 8*(lane/16) .. +7].
__device__ __forceinline__ void load_q(bf16x8 (&qf)[kDqk / 32], const uint16_t* q, int b, int g, int hq, int lane) {
    const u32x4* src = reinterpret_cast<const u32x4*>(q + ((size_t)b * hq + g * kGroup + (lane & 15)) * kDqk);
#pragma unroll
    for (int st = 0; st < kDqk / 32; ++st) qf[st] = __builtin_bit_cast(bf16x8, src[4 * st + (lane >> 4)]);
}

__device__ __forceinline__ void acc_init(WaveAcc& acc) {
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) acc.o[db] = f32x4{};
    acc.m = kNoMax;
    acc.l = 0.0f;
}

__device__ __forceinline__ float sink_log2(const float* sink, int head, bool& has) {
    has = false;
    if (!sink) return kNoMax;
    const float sv = sink[head] * kLog2e;
    if (sv > -__builtin_inff()) {
        has = true;
        return sv;
    }
    return kNoMax;
}

// ---------------------------------------------------------------------------
// Fused RoPE of a decode step (the rotation of the standalone pass, applied to
// the decode kernels' registers).  NoRope stands in for the argument in the
// kernels without it.
struct NoRope {};
template <bool ROPE>
using RopeArg = typename std::conditional<ROPE, DecodeRope, NoRope>::type;

// A lane's frequencies for the angle table, f_lane and f_(lane+64) (rd/2 <=
// 96), loaded once per kernel so that no table waits on them.
struct RopeLane {
    double f0, f1;
};
__device__ __forceinline__ RopeLane rope_lane_freq(const RopeFreq& f, int half, int lane) {
    return RopeLane{lane < half ? f.f[lane] : 0.0, lane + 64 < half ? f.f[lane + 64] : 0.0};
}

// One wave writes the (cos, sin) of the rd/2 angles p * f_i into its own
// table tab[2i], tab[2i + 1]: the angle and its sine and cosine in fp64,
// rounded to fp32, as the standalone pass forms them.
__device__ __forceinline__ void rope_table_wave(float* tab, int p, const RopeLane& fl, int half, int lane) {
    double sn, cs;
    if (lane < half) {
        sincos((double)p * fl.f0, &sn, &cs);
        tab[2 * lane] = (float)cs;
        tab[2 * lane + 1] = (float)sn;
    }
    if (lane + 64 < half) {
        sincos((double)p * fl.f1, &sn, &cs);
        tab[2 * (lane + 64)] = (float)cs;
        tab[2 * (lane + 64) + 1] = (float)sn;
    }
    wave_lds_fence();
}

// 16-byte chunk c (dims 8c .. 8c+7) of a K row after the rotation, from the
// chunk itself and its pair (the chunk rd/16 after it in the first half of the
// rotated dims, before it in the second): x' = x cos - y sin in the first
// half, y' = y cos + x sin in the second (rope_pair's operations), later
// chunks unchanged.
__device__ __forceinline__ u32x4 rope_chunk(const u32x4& own, const u32x4& pair, int c, const float* tab, int half) {
    const int hc = half / 8;
    if (c >= 2 * hc) return own;
    const bool first = c < hc;
    const int i0 = 8 * (first ? c : c - hc);
    const u32x4 x = first ? own : pair, y = first ? pair : own;
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int i = i0 + 2 * w;
        float a0, a1, b0, b1;
        rope_pair(bf16_word_lo(x[w]), bf16_word_lo(y[w]), tab[2 * i], tab[2 * i + 1], a0, b0);
        rope_pair(bf16_word_hi(x[w]), bf16_word_hi(y[w]), tab[2 * i + 2], tab[2 * i + 3], a1, b1);
        o[w] = first ? pack_bf16x2(a0, a1) : pack_bf16x2(b0, b1);
    }
    return o;
}

// The rotation of a merge thread's strided values v[m] = dim jd + 16m of a
// head (q and the new key): with rd/2 = 16 HM the pair of dim d < rd/2 is
// v[m + HM], and each rotated value is rounded to bf16 as the standalone pass
// stores it.
template <int HM>
__device__ __forceinline__ void rope_strided(float (&qv)[kDqk / 16], float (&kv)[kDqk / 16], const float* tab,
                                             int jd) {
    float qr[kDqk / 16], kr[kDqk / 16];
#pragma unroll
    for (int m = 0; m < kDqk / 16; ++m) {
        qr[m] = qv[m];
        kr[m] = kv[m];
    }
#pragma unroll
    for (int m = 0; m < HM; ++m) {
        const int i = jd + 16 * m;
        const float c = tab[2 * i], sn = tab[2 * i + 1];
        float x, y;
        rope_pair(qv[m], qv[m + HM], c, sn, x, y);
        qr[m] = bf16_word_lo(pack_bf16x2(x, 0.0f));
        qr[m + HM] = bf16_word_lo(pack_bf16x2(y, 0.0f));
        rope_pair(kv[m], kv[m + HM], c, sn, x, y);
        kr[m] = bf16_word_lo(pack_bf16x2(x, 0.0f));
        kr[m + HM] = bf16_word_lo(pack_bf16x2(y, 0.0f));
    }
#pragma unroll
    for (int m = 0; m < kDqk / 16; ++m) {
        qv[m] = qr[m];
        kv[m] = kr[m];
    }
}

// ---------------------------------------------------------------------------
// SWA decode: the ring's 32-key tiles go to the 4 waves; the new token joins in
// the merge instead of as a tile of its own (a one-key MFMA tile would double
// the work of the wave holding it): merge thread (local head tid/16, j =
// tid%16) holds dims j + 16m (m < 12) of the head's query and of the new key
// and 8 values of the new value row, and the 16 threads of a head sum the dot
// product.  The stride of 16 keeps each rotated pair (i, i + rd/2 with rd/2 a
// multiple of 32) inside one thread.
// kShortRing: the ring has at most 256 slots, so every wave owns at most two tiles.
// ROPE: q and the new token's k arrive unrotated and rotate at rope.pos[b]
// (with the fused append only); the ring holds rotated keys.
template <bool kShortRing, bool ROPE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(kShortRing ? 2 : 1, kShortRing ? 2 : 1))) void swa_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const uint16_t* __restrict__ ring_k, const uint16_t* __restrict__ ring_v, const int32_t* __restrict__ ctx_lens,
    const float* __restrict__ sink, uint16_t* __restrict__ out, float* __restrict__ lse, int hq, int hkv, int R,
    float c_log2, float value_scale, uint16_t* __restrict__ app_k, uint16_t* __restrict__ app_v,
    const RopeArg<ROPE> rope) {
    // V tiles of the 4 waves, reused afterwards for the cross-wave merge.
    __shared__ __attribute__((aligned(1024))) char lds[kSwaLdsBytes];
    __shared__ __attribute__((aligned(16))) float rtab_all[ROPE ? 4 * kDqk : 4];  // per wave (cos, sin)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.x, g = blockIdx.y;
    const int p = ctx_lens[b];
    const int rowk = hkv * kDqk * 2, rowv = hkv * kDv * 2;
    const int hl = tid >> 4;  // merge: local head 0..15
    const int jd = tid & 15;  // merge: dims jd + 16m of q and k, values 8jd .. 8jd+7
    const int head = g * kGroup + hl;

    // Fused append: this thread's 16 bytes of the new token's K or V row of
    // group g, loaded now and stored once the ring has been read.
    u32x4 app_row = {}, app_pair = {};
    const uint16_t* knew = k_new + ((size_t)b * hkv + g) * kDqk;
    const u32x4* knew_row = reinterpret_cast<const u32x4*>(knew);
    if (app_k && tid < (kDqk + kDv) / 8)
        app_row = tid < kDqk / 8 ? knew_row[tid]
                                 : reinterpret_cast<const u32x4*>(v_new + ((size_t)b * hkv + g) * kDv)[tid - kDqk / 8];
    // The new token's share of this merge thread.
    uint16_t qn[kDqk / 16], kn[kDqk / 16];
    {
        const uint16_t* qrow = q + ((size_t)b * hq + head) * kDqk;
#pragma unroll
        for (int m = 0; m < kDqk / 16; ++m) {
            qn[m] = qrow[jd + 16 * m];
            kn[m] = knew[jd + 16 * m];
        }
    }
    const u32x4 vn = reinterpret_cast<const u32x4*>(v_new + ((size_t)b * hkv + g) * kDv)[jd];
    int hc = 0;  // ROPE: K chunks in the first half of the rotated dims
    RopeLane fl{};
    int rpos = 0;
    if constexpr (ROPE) {
        hc = rope.half / 8;
        if (app_k && tid < 2 * hc) app_pair = knew_row[tid < hc ? tid + hc : tid - hc];
        fl = rope_lane_freq(rope.freq, rope.half, lane);
        rpos = rope.pos[b];
    }
    bf16x8 qf[kDqk / 32];
    load_q(qf, q, b, g, hq, lane);
    // Slot j holds position p-R+((j-p) mod R); all R slots are in the window
    // once p >= R, otherwise slots 0..p-1 are.  The short-ring kernel reads
    // the whole ring without waiting for p (its staging zeroes the rows past
    // nvalid); the long-ring one bounds its descriptors by p.
    const int nring = min(p, R);
    const uint32_t ring_rows = kShortRing ? (uint32_t)R : (uint32_t)nring;
    const rsrc_t rk = make_rsrc(ring_k + (size_t)b * R * hkv * kDqk, ring_rows * rowk);
    const rsrc_t rv = make_rsrc(ring_v + (size_t)b * R * hkv * kDv, ring_rows * rowv);
    const int ring_tiles = (R + kTile - 1) / kTile;
    const int ntiles = (ring_tiles - wave + 3) / 4;  // ring tiles wave, wave+4, ...
    const rsrc_t none = make_rsrc(k_new, 0);
    auto get = [&](int i) -> TileSrc {
        if (i < ntiles) {
            const int rt = wave + 4 * i;
            return TileSrc{rk, rv, rt * kTile * rowk, rt * kTile * rowv, min(max(nring - rt * kTile, 0), kTile)};
        }
        return TileSrc{none, none, 0, 0, 0};
    };
    const LaneOffsets lo = lane_offsets(lane, g, rowk, rowv);
    WaveAcc acc;
    acc_init(acc);
    float* rtab = rtab_all + (ROPE ? wave * kDqk : 0);
    // The new token's score for head hl (log2 domain): 12 products per thread,
    // summed over the 16 threads of the head; formed while the ring tiles load.
    float sv = 0.0f;
    auto new_score = [&]() {
        float qv[kDqk / 16], kv[kDqk / 16];
#pragma unroll
        for (int m = 0; m < kDqk / 16; ++m) {
            qv[m] = __builtin_bit_cast(float, (uint32_t)qn[m] << 16);
            kv[m] = __builtin_bit_cast(float, (uint32_t)kn[m] << 16);
        }
        if constexpr (ROPE) {
            switch (rope.half / 32) {
                case 1: rope_strided<2>(qv, kv, rtab, jd); break;
                case 2: rope_strided<4>(qv, kv, rtab, jd); break;
                case 3: rope_strided<6>(qv, kv, rtab, jd); break;
                default: break;
            }
        }
        float part = 0.0f;
#pragma unroll
        for (int m = 0; m < kDqk / 16; ++m) part = __builtin_fmaf(qv[m], kv[m], part);
        part += __shfl_xor(part, 8);
        part += __shfl_xor(part, 4);
        part += __shfl_xor(part, 2);
        part += __shfl_xor(part, 1);
        sv = part * c_log2;
    };
    if constexpr (ROPE) {
        // Each wave forms the angles while its first tiles load; then q rotates
        // in registers, the new token's q and k values of the merge thread, and
        // (wave 0) the row the fused append writes.
        auto prep = [&]() {
            rope_table_wave(rtab, rpos, fl, rope.half, lane);
            rope_frags32_rd(qf, rtab, rope.half, lane >> 4);
            if (app_k && tid < 2 * hc) app_row = rope_chunk(app_row, app_pair, tid, rtab, rope.half);
            new_score();
        };
        if constexpr (kShortRing)
            run_two_tiles(acc, qf, lds + wave * kVTileBytes, ntiles, get, lo, rowv, c_log2, lane, prep);
        else
            run_tiles<kSwaDepth>(acc, qf, lds + wave * kVTileBytes, ntiles, get, lo, rowv, c_log2, lane, prep);
    } else {
        if constexpr (kShortRing)
            run_two_tiles(acc, qf, lds + wave * kVTileBytes, ntiles, get, lo, rowv, c_log2, lane, new_score);
        else
            run_tiles<kSwaDepth>(acc, qf, lds + wave * kVTileBytes, ntiles, get, lo, rowv, c_log2, lane, new_score);
    }
    acc.l += __shfl_xor(acc.l, 16);
    acc.l += __shfl_xor(acc.l, 32);

    // Merge the 4 waves and the new token: per wave O [16 heads][128 dv] and
    // 16 x (m, l) in fp32.
    __syncthreads();
    float* mrg_o = reinterpret_cast<float*>(lds);     // [wave][16][kMergeRow]
    float* mrg_ml = mrg_o + 4 * kGroup * kMergeRow;   // [wave][16][2]
    const int G = lane >> 4, h = lane & 15;
    if (G == 0) {
        mrg_ml[(wave * kGroup + h) * 2 + 0] = acc.m;
        mrg_ml[(wave * kGroup + h) * 2 + 1] = acc.l;
    }
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db)
        *reinterpret_cast<f32x4*>(mrg_o + (wave * kGroup + h) * kMergeRow + 16 * db + 4 * G) = acc.o[db];
    __syncthreads();
    if (app_k && tid < (kDqk + kDv) / 8) {
        // Fused append: the new token goes to ring slot p mod R.  That slot
        // (position p - R) was read by this workgroup only, and every wave's
        // ring loads were consumed before the barrier above.
        const size_t slot_row = (size_t)b * R + p % R;
        if (tid < kDqk / 8)
            reinterpret_cast<u32x4*>(app_k + (slot_row * hkv + g) * kDqk)[tid] = app_row;
        else
            reinterpret_cast<u32x4*>(app_v + (slot_row * hkv + g) * kDv)[tid - kDqk / 8] = app_row;
    }

    const int e0 = jd * 8;  // 8 output columns
    bool has;
    const float sl = sink_log2(sink, head, has);
    float M = fmaxf(sl, sv);
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg_ml[(w * kGroup + hl) * 2]);
    float Z = has ? fast_exp2(sl - M) : 0.0f;
    float o[8] = {};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float wt = fast_exp2(mrg_ml[(w * kGroup + hl) * 2] - M);
        Z += wt * mrg_ml[(w * kGroup + hl) * 2 + 1];
        const float* src_o = mrg_o + (w * kGroup + hl) * kMergeRow + e0;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += wt * src_o[e];
    }
    const float pn = fast_exp2(sv - M);
    Z += pn;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o[2 * e] += pn * bf16_word_lo(vn[e]);
        o[2 * e + 1] += pn * bf16_word_hi(vn[e]);
    }
    const float inv = value_scale / Z;
    u32x4 w4 = {pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
    *reinterpret_cast<u32x4*>(out + ((size_t)b * hq + head) * kDv + e0) = w4;
    if (lse && (tid & 15) == 0) lse[(size_t)b * hq + head] = (M + __log2f(Z)) * kLn2;
}

// ---------------------------------------------------------------------------
// GA work plan (see ga_chunk_count): every split workgroup derives the unit
// starts of the sequences from ctx_lens itself (256 threads, each summing a
// contiguous run of sequences, one wave scanning the 256 sums), then finds the
// sequence that holds the first unit of its chunk.  Workgroup (0, 0) also
// writes the starts, K and n to the workspace header for the combine kernel.
struct ChunkPlan {
    long long c0, c1;  // units [c0, c1) of the flattened list
    long long s_lo;    // first unit of sequence b_lo
    int b_lo;          // the sequence holding unit c0
    bool empty;        // chunk index >= n: nothing to do
};

// Position of sequence b's new token in its key order, and whether the grid
// covers its context (ctx_lens[b] <= max_ctx).
__device__ __forceinline__ int ga_new_pos(const int32_t* ctx_lens, int b, int max_ctx) {
    const int c = ctx_lens[b];
    return c > max_ctx ? 0 : c;
}

__device__ ChunkPlan ga_plan(const int32_t* __restrict__ ctx_lens, int batch, int max_ctx, int min_units,
                             int max_chunks, int chunk, long long* __restrict__ header) {
    __shared__ long long seg[256];
    __shared__ long long plan_s, plan_k;
    __shared__ int plan_b;
    const int t = threadIdx.x;
    const int per = (batch + 255) / 256;
    const int b0 = min(t * per, batch), b1 = min(b0 + per, batch);
    long long sum = 0;
    for (int b = b0; b < b1; ++b) sum += ga_seq_units(ga_new_pos(ctx_lens, b, max_ctx));
    seg[t] = sum;
    __syncthreads();
    if (t < 64) {
        const long long a0 = seg[4 * t], a1 = seg[4 * t + 1], a2 = seg[4 * t + 2], a3 = seg[4 * t + 3];
        const long long tot = a0 + a1 + a2 + a3;
        long long inc = tot;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const long long y = __shfl_up(inc, d);
            if (t >= d) inc += y;
        }
        const long long ex = inc - tot;
        seg[4 * t] = ex;
        seg[4 * t + 1] = ex + a0;
        seg[4 * t + 2] = ex + a0 + a1;
        seg[4 * t + 3] = ex + a0 + a1 + a2;
        if (t == 63) plan_k = inc;
    }
    __syncthreads();
    const long long K = plan_k;
    const long long n = ga_chunk_count(K, min_units, max_chunks);
    ChunkPlan pl;
    pl.c0 = (long long)chunk * K / n;
    pl.c1 = (long long)(chunk + 1) * K / n;
    pl.empty = chunk >= n;
    long long s = seg[t];
    for (int b = b0; b < b1; ++b) {
        const long long u = ga_seq_units(ga_new_pos(ctx_lens, b, max_ctx));
        if (header) header[b] = s;
        if (!pl.empty && s <= pl.c0 && pl.c0 < s + u) {
            plan_b = b;
            plan_s = s;
        }
        s += u;
    }
    if (header && t == 0) {
        header[batch] = K;
        header[batch + 1] = n;
    }
    __syncthreads();
    pl.b_lo = __builtin_amdgcn_readfirstlane(plan_b);
    pl.s_lo = plan_s;
    return pl;
}

// Writes a wave's partial (m, l, O) of 16 heads to workspace slot `slot`.
__device__ __forceinline__ void store_partial(const WaveAcc& acc, float* ws_ml, float* ws_o, size_t slot, int hq,
                                              int g, int lane) {
    const int G = lane >> 4, h = lane & 15;
    const size_t row = slot * hq + g * kGroup + h;
    if (G == 0) {
        ws_ml[row * 2 + 0] = acc.m;
        ws_ml[row * 2 + 1] = acc.l;
    }
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) *reinterpret_cast<f32x4*>(ws_o + row * kDv + 16 * db + 4 * G) = acc.o[db];
}

// Walks the pieces of a chunk: piece(b, u0, u1, p) gets units [u0, u1) of
// sequence b (pool tiles u < ceil(p/32), then the new-token unit), in order.
template <class Piece>
__device__ __forceinline__ void for_each_piece(const ChunkPlan& pl, const int32_t* ctx_lens, int max_ctx,
                                               const Piece& piece) {
    int b = pl.b_lo;
    long long s = pl.s_lo;
    while (s < pl.c1) {
        const int p = ga_new_pos(ctx_lens, b, max_ctx);
        const long long u = ga_seq_units(p);
        const int u0 = (int)(pl.c0 > s ? pl.c0 - s : 0);
        const int u1 = (int)(pl.c1 - s < u ? pl.c1 - s : u);
        piece(b, u0, u1, p);
        s += u;
        ++b;
    }
}

// Pool keys [k0, kend) of one sequence of a paged pool (tb: its block-table
// row, page_shift = log2 P), in spans of at most kMaxSplitPages pages cut at
// 32-key tile boundaries.  Each span preloads its page numbers, two per lane
// (-1 past the table's end), and calls span(npool, last, pool_tile):
// pool_tile(i) describes the span's i-th 32-key tile through a descriptor per
// 16-key half (each inside one page), with no records for keys past the span
// or on an unmapped block.  Row sizes are in bytes (the bf16 and the FP8 pool
// share this walk).  A span is visited even when it has no pool tile.
template <class Span>
__device__ __forceinline__ void for_each_page_span(const int32_t* __restrict__ tb, int max_blocks, int page_shift,
                                                   long long num_pages, const void* pool_k, const void* pool_v,
                                                   int rowk_bytes, int rowv_bytes, int k0, int kend, int lane,
                                                   const Span& span) {
    const int pmask = (1 << page_shift) - 1;
    int a = k0;
    bool more = true;
    while (more) {
        const int first = a >> page_shift;
        const long long lim = ((long long)(first + kMaxSplitPages) << page_shift) / kTile * kTile;
        const int span_end = (int)(lim < kend ? lim : kend);
        more = span_end < kend;
        const int npool = (span_end - a + kTile - 1) / kTile;
        const int pg_lo = first + lane < max_blocks ? tb[first + lane] : -1;
        const int pg_hi = first + 64 + lane < max_blocks ? tb[first + 64 + lane] : -1;
        // Descriptor of the n valid keys from position j on (inside one page);
        // no records when n <= 0 or the block is unmapped.
        auto half = [&](const void* pool, int row_bytes, int j, int n) -> rsrc_t {
            const int blk = (j >> page_shift) - first;  // 0..127 whenever n > 0
            const int pa = __builtin_amdgcn_readlane(pg_lo, blk & 63);
            const int pb = __builtin_amdgcn_readlane(pg_hi, blk & 63);
            const int pg = (blk & 64) ? pb : pa;
            const bool ok = n > 0 && pg >= 0 && pg < num_pages;
            const size_t row = ((size_t)(ok ? pg : 0) << page_shift) + (size_t)(j & pmask);
            return make_rsrc(static_cast<const char*>(pool) + row * row_bytes, ok ? (uint32_t)n * (uint32_t)row_bytes : 0u);
        };
        const int a0 = a;
        auto pool_tile = [&](int i) -> PagedTileSrc {
            const int j0 = a0 + i * kTile;
            const int n = min(span_end - j0, kTile);
            return PagedTileSrc{{half(pool_k, rowk_bytes, j0, min(n, 16)), half(pool_k, rowk_bytes, j0 + 16, n - 16)},
                                {half(pool_v, rowv_bytes, j0, min(n, 16)), half(pool_v, rowv_bytes, j0 + 16, n - 16)},
                                n};
        };
        span(npool, !more, pool_tile);
        a = span_end;
    }
}

// PAGED: pool rows come through block_table (page_shift = log2 P); otherwise
// sequence b's rows start at kv_base[b].  ROPE (contiguous pool, fused append):
// q and the new token's k arrive unrotated and rotate at rope.pos[b]; each wave
// forms the angles of the sequence of each piece it computes.
template <bool PAGED, bool ROPE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void ga_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const uint16_t* __restrict__ pool_k, const uint16_t* __restrict__ pool_v, const int64_t* __restrict__ kv_base,
    const int32_t* __restrict__ ctx_lens, int batch, int max_ctx, int min_units, int max_chunks, int hq, int hkv,
    float c_log2, long long* __restrict__ header, float* __restrict__ ws_ml, float* __restrict__ ws_o,
    const int32_t* __restrict__ block_table, int max_blocks, int page_shift, long long num_pages,
    uint16_t* __restrict__ app_k, uint16_t* __restrict__ app_v, const int64_t* __restrict__ kv_capacity,
    const RopeArg<ROPE> rope) {
    static_assert(!(PAGED && ROPE), "fused RoPE covers the contiguous pool");
    __shared__ __attribute__((aligned(1024))) char lds[kBlockLdsBytes];
    __shared__ __attribute__((aligned(16))) float rtab_all[ROPE ? 4 * kDqk : 4];  // per wave (cos, sin)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int chunk = blockIdx.x;
    const ChunkPlan pl = ga_plan(ctx_lens, batch, max_ctx, min_units, max_chunks, chunk,
                                 chunk == 0 && blockIdx.z == 0 ? header : nullptr);
    const int g = blockIdx.z * 4 + wave;
    if (pl.empty || g >= hkv) return;
    const int rowk = hkv * kDqk * 2, rowv = hkv * kDv * 2;
    const LaneOffsets lo = lane_offsets(lane, g, rowk, rowv);
    const rsrc_t none = make_rsrc(k_new, 0);
    RopeLane fl{};
    if constexpr (ROPE) fl = rope_lane_freq(rope.freq, rope.half, lane);
    for_each_piece(pl, ctx_lens, max_ctx, [&](int b, int u0, int u1, int p) {
        int rpos = 0;
        if constexpr (ROPE) rpos = rope.pos[b];
        const int npool_units = (p + kTile - 1) / kTile;
        const bool has_new = u1 > npool_units;  // the new-token unit is the sequence's last
        const int k0 = u0 * kTile;
        const int kend = min(min(u1, npool_units) * kTile, p);  // pool keys [k0, kend)
        // Fused append: row kv_base[b] + ctx of KV head g.  No piece of this
        // launch reads that row (the new token comes from k_new / v_new).
        auto append = [&](const float* rtab) {
            if (!PAGED && app_k && has_new && lane < (kDqk + kDv) / 8) {
                const int ctx = ctx_lens[b];
                if (ctx < kv_capacity[b]) {
                    const size_t row = (size_t)kv_base[b] + ctx;
                    const u32x4* knew_row = reinterpret_cast<const u32x4*>(k_new + ((size_t)b * hkv + g) * kDqk);
                    if (lane < kDqk / 8) {
                        u32x4 x = knew_row[lane];
                        if constexpr (ROPE) {
                            const int hc = rope.half / 8;
                            if (lane < 2 * hc)
                                x = rope_chunk(x, knew_row[lane < hc ? lane + hc : lane - hc], lane, rtab, rope.half);
                        }
                        reinterpret_cast<u32x4*>(app_k + (row * hkv + g) * kDqk)[lane] = x;
                    } else {
                        reinterpret_cast<u32x4*>(app_v + (row * hkv + g) * kDv)[lane - kDqk / 8] =
                            reinterpret_cast<const u32x4*>(v_new + ((size_t)b * hkv + g) * kDv)[lane - kDqk / 8];
                    }
                }
            }
        };
        if constexpr (!ROPE) append(nullptr);
        bf16x8 qf[kDqk / 32];
        load_q(qf, q, b, g, hq, lane);
        const rsrc_t nk = make_rsrc(k_new + (size_t)b * hkv * kDqk, (uint32_t)rowk);
        const rsrc_t nv = make_rsrc(v_new + (size_t)b * hkv * kDv, (uint32_t)rowv);
        WaveAcc acc;
        acc_init(acc);
        if constexpr (PAGED) {
            for_each_page_span(block_table + (size_t)b * max_blocks, max_blocks, page_shift, num_pages, pool_k, pool_v,
                               rowk, rowv, k0, kend, lane, [&](int npool, bool last, const auto& pool_tile) {
                const int ntiles = npool + (last && has_new ? 1 : 0);
                auto get = [&](int i) -> PagedTileSrc {
                    if (i < npool) return pool_tile(i);
                    if (i < ntiles) return PagedTileSrc{{nk, none}, {nv, none}, 1};
                    return PagedTileSrc{{none, none}, {none, none}, 0};
                };
                run_tiles<kGaDepth>(acc, qf, lds + wave * kVTileBytes, ntiles, get, lo, rowv, c_log2, lane);
            });
        } else {
            const size_t base = (size_t)kv_base[b];
            const rsrc_t pk = make_rsrc(pool_k + base * hkv * kDqk, (uint32_t)p * rowk);
            const rsrc_t pv = make_rsrc(pool_v + base * hkv * kDv, (uint32_t)p * rowv);
            const int npool = (kend - k0 + kTile - 1) / kTile;
            const int ntiles = npool + (has_new ? 1 : 0);
            auto get = [&](int i) -> TileSrc {
                if (i < npool) {
                    const int j0 = k0 + i * kTile;
                    return TileSrc{pk, pv, j0 * rowk, j0 * rowv, min(kend - j0, kTile)};
                }
                if (i < ntiles) return TileSrc{nk, nv, 0, 0, 1};
                return TileSrc{none, none, 0, 0, 0};
            };
            if constexpr (ROPE) {
                // The wave's angles for sequence b are formed while its first
                // tiles load; the new-token tile is the piece's last.
                float* rtab = rtab_all + wave * kDqk;
                auto prep = [&]() {
                    rope_table_wave(rtab, rpos, fl, rope.half, lane);
                    rope_frags32_rd(qf, rtab, rope.half, lane >> 4);
                    append(rtab);
                };
                const int new_idx = has_new ? npool : -1;
                auto khook = [&](int i, u32x4 (&kr)[12]) {
                    if (i == new_idx) rope_frags32_rd(kr, rtab, rope.half, lane >> 4);
                };
                run_tiles<kGaDepth>(acc, qf, lds + wave * kVTileBytes, ntiles, get, lo, rowv, c_log2, lane, prep,
                                    khook);
            } else {
                run_tiles<kGaDepth>(acc, qf, lds + wave * kVTileBytes, ntiles, get, lo, rowv, c_log2, lane);
            }
        }
        acc.l += __shfl_xor(acc.l, 16);
        acc.l += __shfl_xor(acc.l, 32);
        store_partial(acc, ws_ml, ws_o, (size_t)chunk + b, hq, g, lane);
    });
}

// ---------------------------------------------------------------------------
// FP8 GA pool: OCP E4M3 codes, one fp32 scale per KV head for K and for V, so a
// cached token is 768 B of K and 512 B of V for the 4 heads (half the bf16
// pool).  Codes widen exactly to bf16 in registers (an E4M3 value has at most 4
// significant bits and an exponent inside bf16's range), and
// the bf16 MFMA tile runs on them unchanged; the K scale joins the score
// multiplier, and the V scale multiplies the split's partial output once.  The
// contraction over d is permuted so that one 16-byte load feeds two k-steps:
// k-steps 2u and 2u+1 of lane group G = lane/16 take d = 64u + 16G .. +7 and
// 64u + 16G + 8 .. +15, for K and for Q alike (a dot product does not depend
// on the order of its terms).  The new token (bf16 k_new, v_new) is folded in
// after the cached tiles in fp32, so its weight is not rounded to bf16.

// Lane-constant byte offsets inside an FP8 tile.  K: lane l reads keys l%16
// (and +16), 16 codes at d = 64u + 16(l/16) for u = 0..2.  V: load i reads key
// 8i + l/8, 16 codes at columns 16(l%8) .. +15.
struct Fp8LaneOffsets {
    int k0, k1, v;
};

__device__ __forceinline__ Fp8LaneOffsets fp8_lane_offsets(int lane, int g, int rowk8, int rowv8) {
    Fp8LaneOffsets o;
    o.k0 = (lane & 15) * rowk8 + g * kDqk + (lane >> 4) * 16;
    o.k1 = o.k0 + 16 * rowk8;
    o.v = (lane >> 3) * rowv8 + g * kDv + (lane & 7) * 16;
    return o;
}

__device__ __forceinline__ void issue_k8(const TileSrc& t, const Fp8LaneOffsets& lo, u32x4 (&k)[6]) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        k[u] = __builtin_amdgcn_raw_buffer_load_b128(t.k, lo.k0 + 64 * u, t.koff, 0);
        k[3 + u] = __builtin_amdgcn_raw_buffer_load_b128(t.k, lo.k1 + 64 * u, t.koff, 0);
    }
}

__device__ __forceinline__ void issue_v8(const TileSrc& t, const Fp8LaneOffsets& lo, int rowv8, u32x4 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(t.v, lo.v, t.voff + 8 * i * rowv8, 0);
}

// Paged halves: K rows l%16 of each half; V load i takes key 8i + l/8, i.e.
// half i/2 at row 8(i%2) + l/8.
__device__ __forceinline__ void issue_k8(const PagedTileSrc& t, const Fp8LaneOffsets& lo, u32x4 (&k)[6]) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        k[u] = __builtin_amdgcn_raw_buffer_load_b128(t.k[0], lo.k0 + 64 * u, 0, 0);
        k[3 + u] = __builtin_amdgcn_raw_buffer_load_b128(t.k[1], lo.k0 + 64 * u, 0, 0);
    }
}

__device__ __forceinline__ void issue_v8(const PagedTileSrc& t, const Fp8LaneOffsets& lo, int rowv8, u32x4 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(t.v[i / 2], lo.v, 8 * (i % 2) * rowv8, 0);
}

// V codes to the wave's bf16 LDS tile, in the layout stage_v writes: load i
// holds row r = 8i + l/8, bf16 chunks c = 2(l%8) and c+1, stored at chunk
// positions c ^ 2(r%8) and that + 1 (c is even), i.e. one 32-byte run.
__device__ __forceinline__ void stage_v8(const u32x4 (&v)[4], char* vbuf, int lane) {
    const int r0 = lane >> 3, c0 = 2 * (lane & 7);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + r0;
        char* dst = vbuf + r * (kDv * 2) + ((c0 ^ (2 * r0)) * 16);
        *reinterpret_cast<u32x4*>(dst) = fp8x8_to_bf16x8(v[i][0], v[i][1]);
        *reinterpret_cast<u32x4*>(dst + 16) = fp8x8_to_bf16x8(v[i][2], v[i][3]);
    }
    wave_lds_fence();
}

// K codes to attend_tile's A operands: k-step 2u+h of key block blk comes from
// half h of load 3*blk + u.
__device__ __forceinline__ void widen_k8(const u32x4 (&k8)[6], u32x4 (&kb)[12]) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            kb[6 * blk + 2 * u] = fp8x8_to_bf16x8(k8[3 * blk + u][0], k8[3 * blk + u][1]);
            kb[6 * blk + 2 * u + 1] = fp8x8_to_bf16x8(k8[3 * blk + u][2], k8[3 * blk + u][3]);
        }
}

// Q^T fragments in the permuted contraction order: qf[2u+h] holds
// q[16*g + lane%16][64u + 16(lane/16) + 8h .. +7].
__device__ __forceinline__ void load_q_perm(bf16x8 (&qf)[kDqk / 32], const uint16_t* q, int b, int g, int hq,
                                            int lane) {
    const u32x4* src = reinterpret_cast<const u32x4*>(q + ((size_t)b * hq + g * kGroup + (lane & 15)) * kDqk);
    const int G = lane >> 4;
#pragma unroll
    for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h) qf[2 * u + h] = __builtin_bit_cast(bf16x8, src[8 * u + 2 * G + h]);
}

// As run_tiles, over FP8 tiles (D + 1 register sets of 6 K and 4 V loads).
template <int D, class GetTile>
__device__ __forceinline__ void run_tiles_fp8(WaveAcc& acc, const bf16x8 (&qf)[kDqk / 32], char* vbuf, int ntiles,
                                              const GetTile& get, const Fp8LaneOffsets& lo, int rowv8, float c_log2,
                                              int lane) {
    if (ntiles <= 0) return;
    u32x4 kr[D + 1][6], vr[D + 1][4];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const auto t = get(j);
        issue_k8(t, lo, kr[j]);
        issue_v8(t, lo, rowv8, vr[j]);
    }
    for (int i0 = 0; i0 < ntiles; i0 += D + 1) {
#pragma unroll
        for (int j = 0; j <= D; ++j) {
            const auto t = get(i0 + j + D);
            issue_k8(t, lo, kr[(j + D) % (D + 1)]);
            issue_v8(t, lo, rowv8, vr[(j + D) % (D + 1)]);
            stage_v8(vr[j], vbuf, lane);
            u32x4 kb[12];
            widen_k8(kr[j], kb);
            attend_tile(acc, qf, kb, vbuf, get(i0 + j).nvalid, c_log2, lane);
        }
    }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Folds the new token (bf16 k_new/v_new row of group g) into a wave's state in
// fp32: its score from the permuted Q fragments (each lane a 48-term partial,
// summed over the head's 4 lanes), then one more online-softmax step.  acc.l
// must already be the full (cross-lane) sum.
__device__ __forceinline__ void fold_new_token(WaveAcc& acc, const bf16x8 (&qf)[kDqk / 32], const uint16_t* krow,
                                               const uint16_t* vrow, float c_log2, int lane) {
    const int G = lane >> 4;
    const u32x4* kn = reinterpret_cast<const u32x4*>(krow);
    float dot = 0.0f;
#pragma unroll
    for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4 kw = kn[8 * u + 2 * G + h];
            const u32x4 qw = __builtin_bit_cast(u32x4, qf[2 * u + h]);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                dot += bf16_lo(qw[t]) * bf16_lo(kw[t]) + bf16_hi(qw[t]) * bf16_hi(kw[t]);
        }
    dot += __shfl_xor(dot, 16);
    dot += __shfl_xor(dot, 32);
    const float s = dot * c_log2;
    const float m_new = fmaxf(acc.m, s);
    const float alpha = fast_exp2(acc.m - m_new), pn = fast_exp2(s - m_new);
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) {
        const u32x2 vw = *reinterpret_cast<const u32x2*>(vrow + 16 * db + 4 * G);
        const f32x4 vv = {bf16_lo(vw[0]), bf16_hi(vw[0]), bf16_lo(vw[1]), bf16_hi(vw[1])};
        acc.o[db] = acc.o[db] * alpha + pn * vv;
    }
    acc.l = acc.l * alpha + pn;
    acc.m = m_new;
}

// PAGED: code rows come through block_table, as for the bf16 pool.
template <bool PAGED>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void ga_split_fp8_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const uint8_t* __restrict__ pool_k, const uint8_t* __restrict__ pool_v, const int64_t* __restrict__ kv_base,
    const int32_t* __restrict__ ctx_lens, const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    int batch, int max_ctx, int min_units, int max_chunks, int hq, int hkv, float c_log2,
    long long* __restrict__ header, float* __restrict__ ws_ml, float* __restrict__ ws_o,
    const int32_t* __restrict__ block_table, int max_blocks, int page_shift, long long num_pages) {
    __shared__ __attribute__((aligned(1024))) char lds[kBlockLdsBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int chunk = blockIdx.x;
    const ChunkPlan pl = ga_plan(ctx_lens, batch, max_ctx, min_units, max_chunks, chunk,
                                 chunk == 0 && blockIdx.z == 0 ? header : nullptr);
    const int g = blockIdx.z * 4 + wave;
    if (pl.empty || g >= hkv) return;
    const int rowk8 = hkv * kDqk, rowv8 = hkv * kDv;
    const float ks = k_scale[g], vs = v_scale[g];
    const rsrc_t none = make_rsrc(pool_k, 0);
    const Fp8LaneOffsets lo = fp8_lane_offsets(lane, g, rowk8, rowv8);
    for_each_piece(pl, ctx_lens, max_ctx, [&](int b, int u0, int u1, int p) {
        const int npool_units = (p + kTile - 1) / kTile;
        const bool has_new = u1 > npool_units;
        const int k0 = u0 * kTile;
        const int kend = min(min(u1, npool_units) * kTile, p);  // pool keys [k0, kend)
        bf16x8 qf[kDqk / 32];
        load_q_perm(qf, q, b, g, hq, lane);
        WaveAcc acc;
        acc_init(acc);
        if constexpr (PAGED) {
            for_each_page_span(block_table + (size_t)b * max_blocks, max_blocks, page_shift, num_pages, pool_k, pool_v,
                               rowk8, rowv8, k0, kend, lane, [&](int npool, bool, const auto& pool_tile) {
                auto get = [&](int i) -> PagedTileSrc {
                    if (i < npool) return pool_tile(i);
                    return PagedTileSrc{{none, none}, {none, none}, 0};
                };
                run_tiles_fp8<kFp8Depth>(acc, qf, lds + wave * kVTileBytes, npool, get, lo, rowv8, c_log2 * ks,
                                         lane);
            });
        } else {
            const size_t base = (size_t)kv_base[b];
            const rsrc_t pk = make_rsrc(pool_k + base * rowk8, (uint32_t)p * rowk8);
            const rsrc_t pv = make_rsrc(pool_v + base * rowv8, (uint32_t)p * rowv8);
            const int npool = (kend - k0 + kTile - 1) / kTile;
            auto get = [&](int i) -> TileSrc {
                if (i < npool) {
                    const int j0 = k0 + i * kTile;
                    return TileSrc{pk, pv, j0 * rowk8, j0 * rowv8, min(kend - j0, kTile)};
                }
                return TileSrc{none, none, 0, 0, 0};
            };
            run_tiles_fp8<kFp8Depth>(acc, qf, lds + wave * kVTileBytes, npool, get, lo, rowv8, c_log2 * ks, lane);
        }
        acc.l += __shfl_xor(acc.l, 16);
        acc.l += __shfl_xor(acc.l, 32);
#pragma unroll
        for (int db = 0; db < kDv / 16; ++db) acc.o[db] *= vs;
        if (has_new)
            fold_new_token(acc, qf, k_new + ((size_t)b * hkv + g) * kDqk, v_new + ((size_t)b * hkv + g) * kDv,
                           c_log2, lane);
        store_partial(acc, ws_ml, ws_o, (size_t)chunk + b, hq, g, lane);
    });
}

// Merge of the pieces of one (sequence, head): block (b, head), thread t =
// (piece group t/16, 8 output columns 8(t%16)).  The pieces of sequence b are
// slots first + b .. last + b, first and last being the chunks holding its
// first and last unit (workspace header: unit starts, K, n).  Each thread
// folds the pieces s = t/16, t/16 + 16, ... with an online max (all its loads
// are independent, so they are in flight together), then the 16 groups are
// merged through LDS by the threads of group 0, which add the sink once and
// write the row.
constexpr int kCombGroups = 16;
__global__ __launch_bounds__(256) void ga_combine_kernel(const long long* __restrict__ header,
                                                         const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
                                                         const int32_t* __restrict__ ctx_lens, int batch, int max_ctx,
                                                         const float* __restrict__ sink, uint16_t* __restrict__ out,
                                                         float* __restrict__ lse, int hq, float value_scale) {
    __shared__ float red_ml[kCombGroups][16][2];
    __shared__ __attribute__((aligned(16))) float red_o[kCombGroups][16][8 + 4];  // padded rows
    const int b = blockIdx.x, head = blockIdx.y;
    const int sg = threadIdx.x >> 4, cb = threadIdx.x & 15, e0 = cb * 8;
    uint16_t* orow = out + ((size_t)b * hq + head) * kDv + e0;
    if (ctx_lens[b] > max_ctx) {  // the grid did not cover this context: refuse loudly
        if (sg == 0) {
            *reinterpret_cast<u32x4*>(orow) = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
            if (lse && cb == 0) reinterpret_cast<uint32_t*>(lse)[(size_t)b * hq + head] = 0x7fc00000u;  // quiet NaN bits
        }
        return;
    }
    const long long K = header[batch], n = header[batch + 1];
    const long long s0 = header[b], s1 = header[b + 1];
    const long long first = ((s0 + 1) * n - 1) / K;  // chunk holding unit s0
    const long long last = (s1 * n - 1) / K;         // chunk holding unit s1 - 1
    const int ns = (int)(last - first + 1);
    const size_t row0 = (size_t)(first + b) * hq + head;
    float m = kNoMax, l = 0.0f;
    f32x4 o0 = {}, o1 = {};
    for (int s = sg; s < ns; s += kCombGroups) {
        const size_t row = row0 + (size_t)s * hq;
        const float ms = ws_ml[row * 2], ls = ws_ml[row * 2 + 1];
        const f32x4* src = reinterpret_cast<const f32x4*>(ws_o + row * kDv + e0);
        const f32x4 a0 = src[0], a1 = src[1];
        const float mn = fmaxf(m, ms);
        const float ca = fast_exp2(m - mn), cw = fast_exp2(ms - mn);
        l = l * ca + ls * cw;
        o0 = o0 * ca + a0 * cw;
        o1 = o1 * ca + a1 * cw;
        m = mn;
    }
    red_ml[sg][cb][0] = m;
    red_ml[sg][cb][1] = l;
    *reinterpret_cast<f32x4*>(&red_o[sg][cb][0]) = o0;
    *reinterpret_cast<f32x4*>(&red_o[sg][cb][4]) = o1;
    __syncthreads();
    if (sg != 0) return;
    bool has;
    const float sl = sink_log2(sink, head, has);
    float M = sl;
#pragma unroll
    for (int g = 0; g < kCombGroups; ++g) M = fmaxf(M, red_ml[g][cb][0]);
    float Z = has ? fast_exp2(sl - M) : 0.0f;
    f32x4 t0 = {}, t1 = {};
#pragma unroll
    for (int g = 0; g < kCombGroups; ++g) {
        const float wt = fast_exp2(red_ml[g][cb][0] - M);  // groups without pieces: exp2(kNoMax - M) = 0
        Z += wt * red_ml[g][cb][1];
        t0 += wt * *reinterpret_cast<const f32x4*>(&red_o[g][cb][0]);
        t1 += wt * *reinterpret_cast<const f32x4*>(&red_o[g][cb][4]);
    }
    const float inv = value_scale / Z;
    *reinterpret_cast<u32x4*>(orow) = u32x4{pack_bf16x2(t0[0] * inv, t0[1] * inv), pack_bf16x2(t0[2] * inv, t0[3] * inv),
                                           pack_bf16x2(t1[0] * inv, t1[1] * inv), pack_bf16x2(t1[2] * inv, t1[3] * inv)};
    if (lse && cb == 0) lse[(size_t)b * hq + head] = (M + __log2f(Z)) * kLn2;
}

}  // namespace

hipError_t launch_decode_swa(const DecodeArgs& a, hipStream_t stream) {
    const int R = a.window - 1;
    const bool short_ring = (R + kTile - 1) / kTile <= 8;  // at most two ring tiles per wave
    if (a.rope.pos) {
        auto kern = short_ring ? swa_decode_kernel<true, true> : swa_decode_kernel<false, true>;
        hipLaunchKernelGGL(kern, dim3(a.batch, a.hkv), dim3(256), 0, stream, a.q, a.k_new, a.v_new, a.k_cache, a.v_cache,
                           a.ctx_lens, a.sink, a.out, a.lse, a.hq, a.hkv, R, a.softmax_scale * kLog2e, a.value_scale,
                           a.append_k, a.append_v, a.rope);
        return hipGetLastError();
    }
    auto kern = short_ring ? swa_decode_kernel<true, false> : swa_decode_kernel<false, false>;
    hipLaunchKernelGGL(kern, dim3(a.batch, a.hkv), dim3(256), 0, stream, a.q, a.k_new, a.v_new, a.k_cache, a.v_cache,
                       a.ctx_lens, a.sink, a.out, a.lse, a.hq, a.hkv, R, a.softmax_scale * kLog2e, a.value_scale,
                       a.append_k, a.append_v, NoRope{});
    return hipGetLastError();
}

hipError_t launch_decode_ga(const DecodeArgs& a, hipStream_t stream) {
    const int grid = ga_grid_chunks(a.batch, a.max_ctx, a.min_units, a.max_chunks);
    long long* header = static_cast<long long*>(a.workspace);
    float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + ga_header_bytes(a.batch));
    float* ws_o = ws_ml + (size_t)(grid + a.batch) * a.hq * 2;
    if (a.k_cache8) {
        hipLaunchKernelGGL(a.pages.table ? ga_split_fp8_kernel<true> : ga_split_fp8_kernel<false>,
                           dim3(grid, 1, (a.hkv + 3) / 4), dim3(256), 0, stream, a.q, a.k_new, a.v_new, a.k_cache8,
                           a.v_cache8, a.kv_base, a.ctx_lens, a.k_scale, a.v_scale, a.batch, a.max_ctx, a.min_units,
                           grid, a.hq, a.hkv, a.softmax_scale * kLog2e, header, ws_ml, ws_o, a.pages.table,
                           a.pages.max_blocks, a.pages.shift, a.pages.num_pages);
    } else if (a.rope.pos) {
        auto kern = ga_split_kernel<false, true>;
        hipLaunchKernelGGL(kern, dim3(grid, 1, (a.hkv + 3) / 4), dim3(256), 0, stream, a.q,
                           a.k_new, a.v_new, a.k_cache, a.v_cache, a.kv_base, a.ctx_lens, a.batch, a.max_ctx,
                           a.min_units, grid, a.hq, a.hkv, a.softmax_scale * kLog2e, header, ws_ml, ws_o, nullptr, 0,
                           0, 0LL, a.append_k, a.append_v, a.kv_capacity, a.rope);
    } else {
        auto kern = a.pages.table ? ga_split_kernel<true, false> : ga_split_kernel<false, false>;
        hipLaunchKernelGGL(kern, dim3(grid, 1, (a.hkv + 3) / 4), dim3(256), 0, stream, a.q, a.k_new, a.v_new, a.k_cache,
                           a.v_cache, a.kv_base, a.ctx_lens, a.batch, a.max_ctx, a.min_units, grid, a.hq, a.hkv,
                           a.softmax_scale * kLog2e, header, ws_ml, ws_o, a.pages.table, a.pages.max_blocks,
                           a.pages.shift, a.pages.num_pages, a.pages.table ? nullptr : a.append_k, a.append_v,
                           a.kv_capacity, NoRope{});
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ga_combine_kernel, dim3(a.batch, a.hq), dim3(256), 0, stream, header, ws_ml, ws_o, a.ctx_lens,
                       a.batch, a.max_ctx, a.sink, a.out, a.lse, a.hq, a.value_scale);
    return hipGetLastError();
}

}  // namespace mimo
