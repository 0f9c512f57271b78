// LDS-tiled grouped GEMMs for fp8 weights (E4M3FN with 128x128 fp32 block
// scales, or MXFP8: one E8M0 scale per row and 32 K) and many rows per expert.
//
// The same pipeline as the bf16 LDS-tiled kernels (gemm_large.hip): the
// expert's weight rows are the MFMA M side and the block's tokens the N side;
// operands move global -> LDS with direct-to-LDS loads into two-slot rings,
// group 0 (waves 0..3) loading the weight tile and group 1 (waves 4..7) the
// token tile; each stage is multiplied in two halves with the two waves of a
// SIMD alternating memory and compute phases, one barrier per phase; the K
// walk of a (expert, column tile) starts at a stage keyed by both.  Here a
// workgroup owns 256 weight rows x 128 tokens (block_m = 128): wave w owns
// weight rows 64(w % 4) .. +63 and the 32-token sub-tiles u = w / 4 and
// w / 4 + 2, so each wave holds at most 2 x 2 accumulator tiles and, for the
// block-scaled weights, as many per-stage partial sums.
//
// A stage is K = 128: 128-byte fp8 rows (whole cache lines), one weight scale
// block.  Both operands are dequantised to bf16 in registers
// (v_cvt_scalef32_pk_bf16_fp8, exact: an e4m3 value has 4 significant bits
// and the scale folded into the conversion is a power of two -- the
// activation's group scale, an E8M0 weight scale) and multiplied on the bf16
// matrix cores, so every partial sum is fp32-accurate: GEMM1's results decide
// roundings (bf16 gate/up, the intermediate's fp8 codes), and the fp8 matrix
// cores' dot product drops small products (see the weight-streaming kernels).
// Block-scaled weights: each stage's products are summed apart and added to
// the accumulator times the stage's weight block scale (one fp32 multiply per
// 128-long block, as the weight-streaming fp8 kernels do); MXFP8 weights: the
// E8M0 scales fold into the conversion and the MFMAs accumulate directly.
//
// LDS rows are 128 bytes; chunk c of row r sits at position c ^ ((r >> 1) & 7).
// K16 step t of a stage reads chunk t: 8 bytes at byte 8 (lane / 32) of it,
// the K offset 16 t + 8 (lane / 32) of the bf16 MFMA operand layout (lane l
// holds row l % 32 at K offset (l / 32) * 8).
//
// The block's token-row activation scales (per 128 K, or E8M0 per 32 K) sit in
// an LDS table for the whole K, and so do the tile's block weight scales.
// Packed MXFP8 weight scales arrive with each stage through LDS (one
// direct-to-LDS load of the tile's 16 row groups); row-major ones are read per
// lane, one dword per fragment row and stage.
//
//   GEMM1 (a4+a5): tile = 128 intermediate columns (one quantisation group):
//                  gate rows c0..c0+127 and up rows I+c0..; epilogue a =
//                  bf16(bf16(silu(bf16 g)) * bf16 u), then per row the pow2
//                  scale of its 128-column group (amax across the four waves
//                  through LDS) or of each 32-column group (one wave's
//                  columns), and e4m3 codes (P2 sections 1.1, 1.2).
//   GEMM2 (a6):    tile = 256 output columns h; epilogue y[f] = bf16(tw[f] * acc).
//                  For I <= 256 (one or two stages) a workgroup walks several
//                  column tiles with the token tile resident in LDS
//                  (gemm2_large_q_short_kernel, below).
#include "common.h"

namespace moe {

namespace {

constexpr int kTM = 256;            // weight rows per workgroup
constexpr int kBM = 128;            // tokens per workgroup (= block_m of the alignment)
constexpr int kKB = 128;            // K per stage (fp8 elements = bytes)
constexpr int kRowBytes = kKB;      // 128 bytes per LDS row
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlotA = kTM * kRowBytes;   // 32 KiB
constexpr int kSlotB = kBM * kRowBytes;   // 16 KiB
constexpr int kLoadRows = 1024 / kRowBytes;         // rows one direct-to-LDS load fills
constexpr int kLoadsA = kTM / 4 / kLoadRows;        // weight loads per group-0 wave per stage (8)
constexpr int kLoadsB = kBM / 4 / kLoadRows;        // token loads per group-1 wave per stage (4)
constexpr int kMaxK = 8192;                          // the activation-scale table holds K/32 bytes per row
constexpr int kTabBytes = kBM * (kMaxK / 32);        // 32 KiB
static_assert(2 * (kSlotA + kSlotB) + kTabBytes + kBM * 4 * 4 + 8 * (kMaxK / 128) * 4 + 64 <= 160 * 1024,
              "LDS budget");

typedef __attribute__((address_space(3))) uint8_t lds_t;

__device__ __forceinline__ uint32_t swz_chunk(int row, int chunk) { return uint32_t(chunk ^ ((row >> 1) & 7)) << 4; }
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
__device__ __forceinline__ void barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void load_lds(const uint8_t* gbase, uint32_t off, lds_t* dst) {
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(gbase + off), dst, 16, 0, 0);
}

struct RingQ {
    lds_t* a[2];
    lds_t* b[2];
    const uint32_t* tok;      // byte offset of each token-tile row's source row
    const uint8_t* tscale;    // activation scales of the tile's rows: fp32 per 128 K, or E8M0 bytes per 32 K
    float* part;              // [4][kBM] group amax exchange of the GEMM1 epilogue (block-scaled)
    const float* wscale;      // block-scaled weights: [4 waves][2 fragments][K/128] of the tile's rows
    lds_t* ms[2];             // packed MXFP8 weight scales of a stage: 16 row groups x 64 bytes
};

template <int GEMM, bool MX, int NU>
__device__ __forceinline__ void run_tile_q(const GemmArgs& g, const RingQ& ring, int blk, int tile, int e) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv & 3, grp = wv >> 2;
    const int K = GEMM == 1 ? g.H : g.I;
    const int nst = K / kKB;
    const uint32_t kbytes = uint32_t(K);          // one byte per element
    const int R = g.T * g.topk;

    // ---- load sources (as in the bf16 kernel: load q of a wave fills LDS rows
    //      base + 8 q + i/8, position i % 8, with chunk (i % 8) ^ ((row >> 1) & 7))
    const int lrow = lane >> 3;
    const uint32_t lchunk_even = uint32_t((lane & 7) ^ ((lane >> 4) & 7)) << 4;
    const uint32_t lchunk_odd = uint32_t((lane & 7) ^ (((lane >> 4) + 4) & 7)) << 4;
    const uint8_t* abase;
    const uint8_t* bbase;
    if constexpr (GEMM == 1) {
        abase = static_cast<const uint8_t*>(g.w13) + size_t(e) * 2 * g.I * kbytes;
        bbase = g.xq;
    } else {
        abase = static_cast<const uint8_t*>(g.w2) + (size_t(e) * g.H + size_t(tile) * kTM) * kbytes;
        bbase = static_cast<const uint8_t*>(g.inter) + size_t(blk) * kBM * kbytes;
    }
    // weight row (inside the expert's matrix) of tile row r
    auto weight_row = [&](int r) -> int {
        if constexpr (GEMM == 1) return ((r >> 5) & 1 ? g.I : 0) + tile * 128 + (r >> 6) * 32 + (r & 31);
        else return tile * kTM + r;
    };
    const int rot = (e * 7 + tile) % nst;   // as in the bf16 kernel
    auto kofs = [&](int st) -> uint32_t {
        const int k = st + rot;
        return uint32_t(k < nst ? k : k - nst) * kRowBytes;
    };
    auto kstage = [&](int st) -> int {
        const int k = st + rot;
        return k < nst ? k : k - nst;
    };
    const uint32_t a_lane = uint32_t(lrow) * kbytes;
    auto issue_a = [&](int st, lds_t* A) {   // group 0: 64 weight rows per wave
        const uint8_t* base = abase + kofs(st);
#pragma unroll
        for (int q = 0; q < kLoadsA; ++q) {
            const int r0 = 64 * wm + kLoadRows * q;
            const int grow0 = GEMM == 1 ? weight_row(r0) : r0;   // GEMM2: abase is at the tile's first row
            load_lds(base + size_t(grow0) * kbytes, a_lane + ((q & 1) ? lchunk_odd : lchunk_even), A + r0 * kRowBytes);
        }
    };
    auto issue_b = [&](int st, lds_t* B) {   // group 1: 32 token rows per wave
        const uint8_t* base = bbase + kofs(st);
#pragma unroll
        for (int q = 0; q < kLoadsB; ++q) {
            const int row = 32 * wm + kLoadRows * q + lrow;
            load_lds(base, ring.tok[row] + ((q & 1) ? lchunk_odd : lchunk_even), B + (row - lrow) * kRowBytes);
        }
    };

    // ---- fragment addresses: K16 step t reads 8 bytes of chunk t ------------------
    const int fr = lane & 31;
    const int fk = lane >> 5;
    uint32_t coff[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) coff[t] = swz_chunk(fr, t) + 8 * fk;   // the swizzle of rows 32j + fr: same for all
    const uint32_t a_row = uint32_t(64 * wm + fr) * kRowBytes;        // + 32 rows for the up rows (a = 1)
    const uint32_t b_row = uint32_t(32 * grp + fr) * kRowBytes;       // + 64 rows for the second sub-tile

    // ---- scales ----------------------------------------------------------------
    // block-scaled weights: one fp32 per (128-row block, stage) for each A
    // fragment, from the tile's LDS table
    const int kbn = K / 128;                 // weight scale blocks along K
    const int rows_total = GEMM == 1 ? 2 * g.I : g.H;
    auto wscale = [&](int a, int st) -> float { return ring.wscale[(wm * 2 + a) * kbn + kstage(st)]; };
    // MXFP8 weights: E8M0 bytes of the fragment rows, 4 per stage (one per 32 K)
    const uint8_t* wmx = static_cast<const uint8_t*>(GEMM == 1 ? g.w13_scale : g.w2_scale);
    int mrow[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) mrow[a] = GEMM == 1 ? weight_row(64 * wm + 32 * a + fr) : tile * kTM + 64 * wm + 32 * a + fr;
    const int kb32 = K / 32;
    auto mx_weight_scales = [&](int a, int st) -> uint32_t {   // 4 bytes, block 4k + j in byte j
        const int ks = kstage(st);
        const size_t row = size_t(e) * rows_total + mrow[a];
        if (g.mx_packed) {
            // moe_pack_mx_scales layout: per 16-row group, per 128-K step, lane g*16 + r
            const uint8_t* p = wmx + ((row >> 4) * (K / 128) + ks) * 64 + (row & 15);
            return uint32_t(p[0]) | (uint32_t(p[16]) << 8) | (uint32_t(p[32]) << 16) | (uint32_t(p[48]) << 24);
        }
        return *reinterpret_cast<const uint32_t*>(wmx + row * kb32 + 4 * ks);
    };
    // activation scales from the LDS table: fp32 per (row, 128 K) or E8M0 bytes per (row, 32 K)
    auto tscale_f32 = [&](int u, int st) -> float {
        const int row = 32 * (2 * u + grp) + fr;
        return reinterpret_cast<const float*>(ring.tscale)[row * kbn + kstage(st)];
    };
    auto tscale_mx = [&](int u, int st) -> uint32_t {
        const int row = 32 * (2 * u + grp) + fr;
        return *reinterpret_cast<const uint32_t*>(ring.tscale + row * kb32 + 4 * kstage(st));
    };

    f32x16 acc[2][NU > 0 ? NU : 1];
    f32x16 tmp[2][(NU > 0 && !MX) ? NU : 1];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int u = 0; u < (NU > 0 ? NU : 1); ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][u][i] = 0.0f;
    i32x2 af[2][4], bfr[NU > 0 ? NU : 1][4];
    float sa[2] = {1.0f, 1.0f};                                   // block-scaled: this stage's weight scales
    uint32_t ma[2] = {0, 0}, ma_next[2] = {0, 0};                 // MXFP8: E8M0 bytes of the A rows
    float sb[NU > 0 ? NU : 1];                                    // block-scaled: token scales of the stage
    uint32_t mb[NU > 0 ? NU : 1];                                 // MXFP8: token E8M0 bytes of the stage

    typedef const __attribute__((address_space(3))) i32x2 lds_v2;
    auto read_half = [&](const lds_t* A, const lds_t* B, int h) {
        if constexpr (NU > 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t c = coff[4 * h + j];
#pragma unroll
                for (int a = 0; a < 2; ++a) af[a][j] = *reinterpret_cast<lds_v2*>(A + a_row + c + a * 32 * kRowBytes);
#pragma unroll
                for (int u = 0; u < NU; ++u) bfr[u][j] = *reinterpret_cast<lds_v2*>(B + b_row + c + u * 64 * kRowBytes);
            }
        }
    };
    auto compute = [&](int h) {
        if constexpr (NU > 0) {
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 4 * h + j;   // K16 step inside the stage; MX block t / 2
                bf16x8 av[2], bv[NU];
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const float s = MX ? e8m0_to_f32((ma[a] >> (8 * (t >> 1))) & 0xff) : 1.0f;
                    av[a] = e4m3x8_to_bf16(af[a][j][0], af[a][j][1], s);
                }
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    const float s = MX ? e8m0_to_f32((mb[u] >> (8 * (t >> 1))) & 0xff) : sb[u];
                    bv[u] = e4m3x8_to_bf16(bfr[u][j][0], bfr[u][j][1], s);
                }
#pragma unroll
                for (int u = 0; u < NU; ++u)
#pragma unroll
                    for (int a = 0; a < 2; ++a) {
                        if constexpr (MX) {
                            acc[a][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[u], acc[a][u], 0, 0, 0);
                        } else {
                            if (t == 0) tmp[a][u] = f32x16{};
                            tmp[a][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[u], tmp[a][u], 0, 0, 0);
                        }
                    }
            }
            __builtin_amdgcn_s_setprio(0);
        }
    };
    // the stage's block scales applied to its partial sums
    auto fold = [&]() {
        if constexpr (!MX && NU > 0) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int u = 0; u < NU; ++u)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[a][u][i] = __fadd_rn(acc[a][u][i], __fmul_rn(sa[a], tmp[a][u][i]));
        }
    };
    auto scales_for = [&](int st) {   // MXFP8 row-major scales: this wave's of stage st (into ma_next)
        if constexpr (NU > 0 && MX) {
            if (!g.mx_packed) {
#pragma unroll
                for (int a = 0; a < 2; ++a) ma_next[a] = mx_weight_scales(a, st);
            }
        }
    };
    // Packed MXFP8 scales (moe_pack_mx_scales: per 16-row group and K step of
    // 128, 64 bytes = 4 blocks of 32 K x 16 rows) go through LDS: the tile's 16
    // row groups of a stage are one direct-to-LDS load by wave 0, lane i
    // fetching block i % 4 of group i / 4.  LDS group index of a fragment row:
    // GEMM1 8 a + 2 wm + fr / 16 (gate groups first, then up), GEMM2
    // 4 wm + 2 a + fr / 16.
    auto issue_ms = [&](int st, lds_t* M) {
        if constexpr (MX) {
            if (g.mx_packed && wv == 0) {
                const int gi = lane >> 2;
                const int grow = GEMM == 1 ? ((gi >> 3) ? g.I / 16 : 0) + tile * 8 + (gi & 7) : tile * 16 + gi;
                const size_t rg = size_t(e) * (rows_total / 16) + grow;
                load_lds(wmx + (rg * (K / 128) + kstage(st)) * 64, uint32_t(lane & 3) * 16, M);
            }
        }
    };
    auto read_ms = [&](const lds_t* M) {
        if constexpr (NU > 0 && MX) {
            if (g.mx_packed) {
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const int gi = GEMM == 1 ? 8 * a + 2 * wm + (fr >> 4) : 4 * wm + 2 * a + (fr >> 4);
                    const lds_t* q = M + gi * 64 + (fr & 15);
                    ma[a] = uint32_t(q[0]) | (uint32_t(q[16]) << 8) | (uint32_t(q[32]) << 16) |
                            (uint32_t(q[48]) << 24);
                }
            }
        }
    };
    auto token_scales = [&](int st) {
        if constexpr (NU > 0) {
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if constexpr (MX) mb[u] = tscale_mx(u, st);
                else sb[u] = tscale_f32(u, st);
            }
            if constexpr (!MX) {
#pragma unroll
                for (int a = 0; a < 2; ++a) sa[a] = wscale(a, st);
            }
        }
    };

    auto stage = [&](int s, const lds_t* A, const lds_t* B, lds_t* An, lds_t* Bn, const lds_t* M, lds_t* Mn) {
        const bool more = s + 1 < nst;
        // memory phase, first half: fragments and scales of this stage, the next stage's loads
        if constexpr (MX) {
            if (!g.mx_packed) {
#pragma unroll
                for (int a = 0; a < 2; ++a) ma[a] = ma_next[a];
            }
        }
        read_ms(M);
        read_half(A, B, 0);
        token_scales(s);
        if (more) {
            if (grp == 0) {
                issue_a(s + 1, An);
                issue_ms(s + 1, Mn);
            } else {
                issue_b(s + 1, Bn);
            }
            scales_for(s + 1);
        }
        wait_lgkm0();
        barrier();
        compute(0);
        barrier();
        read_half(A, B, 1);
        wait_lgkm0();
        if (grp == 1) wait_vm0();   // its token loads (and scales) of the next stage
        barrier();
        compute(1);
        fold();
        if (grp == 0) wait_vm0();   // its weight loads (and scales) of the next stage
        barrier();
    };

    if (grp == 0) {
        issue_a(0, ring.a[0]);
        issue_ms(0, ring.ms[0]);
    } else {
        issue_b(0, ring.b[0]);
    }
    scales_for(0);
    wait_vm0();
    barrier();
    if (grp == 1) barrier();   // group 1 runs one phase behind group 0
    for (int s = 0; s < nst; s += 2) {
        stage(s, ring.a[0], ring.b[0], ring.a[1], ring.b[1], ring.ms[0], ring.ms[1]);
        if (s + 1 < nst) stage(s + 1, ring.a[1], ring.b[1], ring.a[0], ring.b[0], ring.ms[1], ring.ms[0]);
    }
    if (grp == 0) barrier();

    // ---- epilogues: sub-tile u sits at token rows (2u + grp) * 32 ---------------
    if constexpr (GEMM == 1) {
        // a for this lane's 16 columns of each live sub-tile; columns
        // tile*128 + 32 wm + (i/4)*8 + 4 fk + i%4
        float av[NU > 0 ? NU : 1][16];
        float amax[NU > 0 ? NU : 1];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int row = blk * kBM + (2 * u + grp) * 32 + fr;
            const float w_in = gemm1_row_weight(g, g.sorted_ids[row]);
            float m_ = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                av[u][i] = swiglu_bf16(acc[0][u][i], acc[1][u][i], w_in, g.clamp, g.clamp_limit);
                m_ = fmaxf(m_, __builtin_fabsf(av[u][i]));
            }
            amax[u] = fmaxf(m_, __shfl_xor(m_, 32));   // the wave's 32 columns of the row
        }
        uint8_t* out = static_cast<uint8_t*>(g.inter);
        if constexpr (!MX) {
            // the 128-column group spans the four waves of the token's group
            if (NU > 0 && fk == 0) {
#pragma unroll
                for (int u = 0; u < NU; ++u) ring.part[wm * kBM + (2 * u + grp) * 32 + fr] = amax[u];
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int tr = (2 * u + grp) * 32 + fr;
                amax[u] = fmaxf(fmaxf(ring.part[tr], ring.part[kBM + tr]),
                                fmaxf(ring.part[2 * kBM + tr], ring.part[3 * kBM + tr]));
            }
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int row = blk * kBM + (2 * u + grp) * 32 + fr;
            const float s = fp8_group_scale(amax[u]);
            const float inv_s = __fdiv_rn(1.0f, s);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t packed = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) packed |= fp8_quant(av[u][q * 4 + j], inv_s) << (8 * j);
                const int col = tile * 128 + wm * 32 + q * 8 + fk * 4;
                *reinterpret_cast<uint32_t*>(out + int64_t(row) * g.I + col) = packed;
            }
            if (fk == 0) {
                if constexpr (MX) {
                    reinterpret_cast<uint8_t*>(g.inter_scale)[int64_t(row) * (g.I / 32) + tile * 4 + wm] =
                        uint8_t(__float_as_uint(s) >> 23);
                } else if (wm == 0) {
                    g.inter_scale[int64_t(row) * (g.I / 128) + tile] = s;
                }
            }
        }
    } else {
        const int hw = tile * kTM + wm * 64;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int f = g.sorted_ids[blk * kBM + (2 * u + grp) * 32 + fr];
            if (f >= R) continue;
            const float tw = gemm2_row_weight(g, f);
            const int64_t yrow = int64_t(f) * g.H;
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f32x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = __fmul_rn(acc[a][u][q * 4 + j], tw);
                    store_y4<true>(g.y, yrow + hw + a * 32 + q * 8 + fk * 4, v);
                }
        }
    }
}

template <int GEMM, bool MX>
__global__ __launch_bounds__(kThreads, 1) void gemm_large_q_kernel(GemmArgs g, int ntiles) {
    __shared__ __attribute__((aligned(1024))) uint8_t sa0[kSlotA], sa1[kSlotA];
    __shared__ __attribute__((aligned(1024))) uint8_t sb0[kSlotB], sb1[kSlotB];
    __shared__ __attribute__((aligned(16))) uint8_t s_tscale[kTabBytes];
    __shared__ uint32_t s_tok[kBM];
    __shared__ float s_part[4 * kBM];
    __shared__ float s_wscale[4 * 2 * (kMaxK / 128)];
    __shared__ __attribute__((aligned(1024))) uint8_t sm0[MX ? 1024 : 16], sm1[MX ? 1024 : 16];
    __shared__ int s_valid;
    const RingQ ring{{(lds_t*)sa0, (lds_t*)sa1}, {(lds_t*)sb0, (lds_t*)sb1}, s_tok, s_tscale, s_part, s_wscale,
                     {(lds_t*)sm0, (lds_t*)sm1}};

    int blk, tile;
    if (!map_active_tile<true>(g, ntiles, blk, tile)) return;
    const int e = __builtin_amdgcn_readfirstlane(g.expert_ids[blk]);
    if (e < 0) return;

    const int R = g.T * g.topk;
    const int K = GEMM == 1 ? g.H : g.I;
    // the token tile's source rows (padding rows read a real row of the block,
    // never stored) and their activation scales
    {
        const int first = g.sorted_ids[blk * kBM];
        const int sbytes = MX ? K / 32 : (K / 128) * 4;   // scale bytes per row
        for (int r = threadIdx.x >> 2; r < kBM; r += kThreads / 4) {
            const int f = g.sorted_ids[blk * kBM + r];
            const int src = GEMM == 1 ? (f < R ? f : first) / g.topk : (f < R ? blk * kBM + r : blk * kBM);
            if ((threadIdx.x & 3) == 0) s_tok[r] = uint32_t(GEMM == 1 ? src : src - blk * kBM) * uint32_t(K);
            const uint8_t* srcs = GEMM == 1 ? reinterpret_cast<const uint8_t*>(g.xs) + size_t(src) * sbytes
                                            : reinterpret_cast<const uint8_t*>(g.inter_scale) + size_t(src) * sbytes;
            for (int b = (threadIdx.x & 3) * 4; b < sbytes; b += 16)
                *reinterpret_cast<uint32_t*>(s_tscale + r * sbytes + b) = *reinterpret_cast<const uint32_t*>(srcs + b);
        }
    }
    if constexpr (!MX) {
        // block scales of the tile's weight rows: wave w' fragment a covers the
        // 128-row block of GEMM1's gate (a = 0) or up (a = 1) rows, or of GEMM2's
        // rows 64 w' ..
        const int kbn = K / 128;
        const int rows_total = GEMM == 1 ? 2 * g.I : g.H;
        const float* wsc = static_cast<const float*>(GEMM == 1 ? g.w13_scale : g.w2_scale);
        for (int idx = threadIdx.x; idx < 4 * 2 * kbn; idx += kThreads) {
            const int w_ = idx / (2 * kbn), a = (idx / kbn) & 1, kb = idx % kbn;
            const int sblk = GEMM == 1 ? (a ? g.I / 128 + tile : tile) : 2 * tile + (w_ >> 1);
            s_wscale[idx] = wsc[(size_t(e) * (rows_total / 128) + sblk) * kbn + kb];
        }
    }
    if (threadIdx.x < 64) {
        int n = 0;
#pragma unroll
        for (int q = 0; q < kBM / 64; ++q) n += __popcll(__ballot(g.sorted_ids[blk * kBM + q * 64 + threadIdx.x] < R));
        if (threadIdx.x == 0) s_valid = n;
    }
    __syncthreads();
    const int live = (s_valid + 31) >> 5;
    const int grp = (threadIdx.x >> 6) >> 2;
    const int nu = (live - grp + 1) >> 1;
    switch (nu) {
        case 0: run_tile_q<GEMM, MX, 0>(g, ring, blk, tile, e); break;
        case 1: run_tile_q<GEMM, MX, 1>(g, ring, blk, tile, e); break;
        default: run_tile_q<GEMM, MX, 2>(g, ring, blk, tile, e); break;
    }
}

// ---- GEMM2 over a short K (I <= 256: one or two stages) -----------------------
// A workgroup with one column tile would spend most of its life on its
// prologue and its y stores with no weight bytes in flight (two stages of
// K = 128).  Here a workgroup keeps the block's token tile in LDS (one slot per
// K stage, loaded once by group 1) and walks `ntw` adjacent column tiles.
// Group 0 streams each tile's weights through the two weight slots; group 1
// multiplies and stores token sub-tiles 0 and 1 and loads nothing after the
// prologue, so its y stores never sit in front of a wait for weights (stores
// count in the same vmcnt as loads).  With every wave loading and storing the
// down GEMM took 100 / 355 us at 1024 / 8192 tokens of the fp8 layer, with
// this split 97 / 343 us; a timing-only copy without the y stores 56 / 159 us,
// and y rows staged through LDS into whole 128-byte lines ran slower (105 /
// 411 us).  Group 0 multiplies sub-tiles 2 and 3 when a block has more than
// 64 rows.
// Same phases and barriers as run_tile_q.
constexpr int kShortK = 256;
constexpr int kShortMaxTiles = kMaxK / kTM;   // column tiles of the widest H

template <bool MX, int NST, int NU>
__device__ __forceinline__ void run_tiles_q2(const GemmArgs& g, const RingQ& ring, int blk, int tile0, int ntw,
                                             int e) {
    static_assert(NST == 1 || NST == 2, "short K: one or two stages");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv & 3, grp = wv >> 2;
    const int K = NST * kKB;
    const uint32_t kbytes = uint32_t(K);
    const int R = g.T * g.topk;
    const int S = ntw * NST;

    const int lrow = lane >> 3;
    const uint32_t lchunk_even = uint32_t((lane & 7) ^ ((lane >> 4) & 7)) << 4;
    const uint32_t lchunk_odd = uint32_t((lane & 7) ^ (((lane >> 4) + 4) & 7)) << 4;
    const uint8_t* wbase = static_cast<const uint8_t*>(g.w2) + (size_t(e) * g.H + size_t(tile0) * kTM) * kbytes;
    const uint8_t* bbase = static_cast<const uint8_t*>(g.inter) + size_t(blk) * kBM * kbytes;
    const uint32_t a_lane = uint32_t(lrow) * kbytes;
    auto issue_a = [&](int s, lds_t* A) {   // group 0: 64 weight rows per wave of stage s
        const int c = NST == 2 ? s >> 1 : s, k = s - c * NST;
        const uint8_t* base = wbase + size_t(c) * kTM * kbytes + k * kRowBytes;
#pragma unroll
        for (int q = 0; q < kLoadsA; ++q) {
            const int r0 = 64 * wm + kLoadRows * q;
            load_lds(base + size_t(r0) * kbytes, a_lane + ((q & 1) ? lchunk_odd : lchunk_even), A + r0 * kRowBytes);
        }
    };
    auto issue_b = [&](int k, lds_t* B) {   // group 1: 32 token rows per wave of K stage k
        const uint8_t* base = bbase + k * kRowBytes;
#pragma unroll
        for (int q = 0; q < kLoadsB; ++q) {
            const int row = 32 * wm + kLoadRows * q + lrow;
            load_lds(base, ring.tok[row] + ((q & 1) ? lchunk_odd : lchunk_even), B + (row - lrow) * kRowBytes);
        }
    };

    const int fr = lane & 31;
    const int fk = lane >> 5;
    uint32_t coff[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) coff[t] = swz_chunk(fr, t) + 8 * fk;
    const uint32_t a_row = uint32_t(64 * wm + fr) * kRowBytes;
    // sub-tile u of a wave: token rows 32 st0 + 32 u .. (group 1 takes
    // sub-tiles 0 and 1, group 0 sub-tiles 2 and 3)
    const int st0 = grp == 1 ? 0 : 2;
    const uint32_t b_row = uint32_t(32 * st0 + fr) * kRowBytes;

    // scales: block-scaled weights from the workgroup's LDS table [tile][128-row block][K stage];
    // MXFP8 weights per lane (E8M0 bytes of the fragment rows, 4 per stage)
    const uint8_t* wmx = static_cast<const uint8_t*>(g.w2_scale);
    auto mx_weight_scales = [&](int a, int s) -> uint32_t {
        const int c = NST == 2 ? s >> 1 : s, k = s - c * NST;
        const size_t row = size_t(e) * g.H + size_t(tile0 + c) * kTM + 64 * wm + 32 * a + fr;
        if (g.mx_packed) {
            const uint8_t* p = wmx + ((row >> 4) * NST + k) * 64 + (row & 15);
            return uint32_t(p[0]) | (uint32_t(p[16]) << 8) | (uint32_t(p[32]) << 16) | (uint32_t(p[48]) << 24);
        }
        return *reinterpret_cast<const uint32_t*>(wmx + row * (K / 32) + 4 * k);
    };

    f32x16 acc[2][NU > 0 ? NU : 1];
    f32x16 tmp[2][(NU > 0 && !MX) ? NU : 1];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int u = 0; u < (NU > 0 ? NU : 1); ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][u][i] = 0.0f;
    i32x2 af[2][4], bfr[NU > 0 ? NU : 1][4];
    float sa = 1.0f;
    uint32_t ma[2] = {0, 0}, ma_next[2] = {0, 0};
    float sb[NU > 0 ? NU : 1];
    uint32_t mb[NU > 0 ? NU : 1];
    // the rows this lane stores, for every tile
    int fo[NU > 0 ? NU : 1];
    float two[NU > 0 ? NU : 1];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        fo[u] = g.sorted_ids[blk * kBM + (st0 + u) * 32 + fr];
        two[u] = fo[u] < R ? gemm2_row_weight(g, fo[u]) : 0.0f;
    }

    typedef const __attribute__((address_space(3))) i32x2 lds_v2;
    auto read_half = [&](const lds_t* A, const lds_t* B, int h) {
        if constexpr (NU > 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t c = coff[4 * h + j];
#pragma unroll
                for (int a = 0; a < 2; ++a) af[a][j] = *reinterpret_cast<lds_v2*>(A + a_row + c + a * 32 * kRowBytes);
#pragma unroll
                for (int u = 0; u < NU; ++u) bfr[u][j] = *reinterpret_cast<lds_v2*>(B + b_row + c + u * 32 * kRowBytes);
            }
        }
    };
    auto compute = [&](int h) {
        if constexpr (NU > 0) {
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 4 * h + j;
                bf16x8 av[2], bv[NU];
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const float s = MX ? e8m0_to_f32((ma[a] >> (8 * (t >> 1))) & 0xff) : 1.0f;
                    av[a] = e4m3x8_to_bf16(af[a][j][0], af[a][j][1], s);
                }
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    const float s = MX ? e8m0_to_f32((mb[u] >> (8 * (t >> 1))) & 0xff) : sb[u];
                    bv[u] = e4m3x8_to_bf16(bfr[u][j][0], bfr[u][j][1], s);
                }
#pragma unroll
                for (int u = 0; u < NU; ++u)
#pragma unroll
                    for (int a = 0; a < 2; ++a) {
                        if constexpr (MX) {
                            acc[a][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[u], acc[a][u], 0, 0, 0);
                        } else {
                            if (t == 0) tmp[a][u] = f32x16{};
                            tmp[a][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[u], tmp[a][u], 0, 0, 0);
                        }
                    }
            }
            __builtin_amdgcn_s_setprio(0);
        }
    };
    auto fold = [&]() {
        if constexpr (!MX && NU > 0) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int u = 0; u < NU; ++u)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[a][u][i] = __fadd_rn(acc[a][u][i], __fmul_rn(sa, tmp[a][u][i]));
        }
    };
    auto scales_for = [&](int s) {   // row-major MXFP8 scales: per lane, one stage ahead
        if constexpr (NU > 0 && MX) {
            if (!g.mx_packed) {
#pragma unroll
                for (int a = 0; a < 2; ++a) ma_next[a] = mx_weight_scales(a, s);
            }
        }
    };
    // packed MXFP8 scales through LDS, as in run_tile_q (GEMM2 group order)
    auto issue_ms = [&](int s, lds_t* M) {
        if constexpr (MX) {
            if (g.mx_packed && wv == 0) {
                const int c = NST == 2 ? s >> 1 : s, k = s - c * NST;
                const size_t rg = (size_t(e) * g.H + size_t(tile0 + c) * kTM) / 16 + (lane >> 2);
                load_lds(wmx + (rg * NST + k) * 64, uint32_t(lane & 3) * 16, M);
            }
        }
    };
    auto read_ms = [&](const lds_t* M) {
        if constexpr (NU > 0 && MX) {
            if (g.mx_packed) {
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const lds_t* q = M + (4 * wm + 2 * a + (fr >> 4)) * 64 + (fr & 15);
                    ma[a] = uint32_t(q[0]) | (uint32_t(q[16]) << 8) | (uint32_t(q[32]) << 16) |
                            (uint32_t(q[48]) << 24);
                }
            }
        }
    };
    auto stage_scales = [&](int s) {
        if constexpr (NU > 0) {
            const int c = NST == 2 ? s >> 1 : s, k = s - c * NST;
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int row = 32 * (st0 + u) + fr;
                if constexpr (MX) mb[u] = *reinterpret_cast<const uint32_t*>(ring.tscale + row * (K / 32) + 4 * k);
                else sb[u] = reinterpret_cast<const float*>(ring.tscale)[row * NST + k];
            }
            if constexpr (!MX) sa = ring.wscale[(c * 2 + (wm >> 1)) * NST + k];
        }
    };
    auto store_tile = [&](int c) {
        if constexpr (NU > 0) {
            const int hw = (tile0 + c) * kTM + wm * 64;
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if (fo[u] < R) {
                    const int64_t yrow = int64_t(fo[u]) * g.H;
#pragma unroll
                    for (int a = 0; a < 2; ++a)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            f32x4 v;
#pragma unroll
                            for (int j = 0; j < 4; ++j) v[j] = __fmul_rn(acc[a][u][q * 4 + j], two[u]);
                            store_y4<true>(g.y, yrow + hw + a * 32 + q * 8 + fk * 4, v);
                        }
                }
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[a][u][i] = 0.0f;
            }
        }
    };

    auto stage = [&](int s, const lds_t* A, const lds_t* B, lds_t* An, const lds_t* M, lds_t* Mn) {
        const bool more = s + 1 < S;
        if constexpr (MX) {
            if (!g.mx_packed) {
#pragma unroll
                for (int a = 0; a < 2; ++a) ma[a] = ma_next[a];
            }
        }
        read_ms(M);
        read_half(A, B, 0);
        stage_scales(s);
        if (more) {
            if (grp == 0) {
                issue_a(s + 1, An);
                issue_ms(s + 1, Mn);
            }
            scales_for(s + 1);
        }
        wait_lgkm0();
        barrier();
        compute(0);
        barrier();
        read_half(A, B, 1);
        wait_lgkm0();
        barrier();
        compute(1);
        fold();
        if (grp == 0) wait_vm0();   // the weights (and scales) of the next stage
        barrier();
    };

    if (grp == 0) {
        issue_a(0, ring.a[0]);
        issue_ms(0, ring.ms[0]);
    } else {
        issue_b(0, ring.b[0]);
        if constexpr (NST == 2) issue_b(1, ring.b[1]);
    }
    scales_for(0);
    wait_vm0();
    barrier();
    if (grp == 1) barrier();   // group 1 runs one phase behind group 0
    for (int s = 0; s < S; s += 2) {
        // S is even when NST == 2; with NST == 1 the last pair may be a single stage
        if constexpr (NST == 2) {
            stage(s, ring.a[0], ring.b[0], ring.a[1], ring.ms[0], ring.ms[1]);
            stage(s + 1, ring.a[1], ring.b[1], ring.a[0], ring.ms[1], ring.ms[0]);
            store_tile(s >> 1);
        } else {
            stage(s, ring.a[0], ring.b[0], ring.a[1], ring.ms[0], ring.ms[1]);
            store_tile(s);
            if (s + 1 < S) {
                stage(s + 1, ring.a[1], ring.b[0], ring.a[0], ring.ms[1], ring.ms[0]);
                store_tile(s + 1);
            }
        }
    }
    if (grp == 0) barrier();
}

template <bool MX, int NST>
__global__ __launch_bounds__(kThreads, 1) void gemm2_large_q_short_kernel(GemmArgs g, int ngroups, int ntw) {
    __shared__ __attribute__((aligned(1024))) uint8_t sa0[kSlotA], sa1[kSlotA];
    __shared__ __attribute__((aligned(1024))) uint8_t sb0[kSlotB], sb1[NST == 2 ? kSlotB : 1024];
    __shared__ __attribute__((aligned(16))) uint8_t s_tscale[kBM * 8];   // 8 bytes per row for K <= 256
    __shared__ uint32_t s_tok[kBM];
    __shared__ float s_wscale[kShortMaxTiles * 2 * NST];
    __shared__ __attribute__((aligned(1024))) uint8_t sm0[MX ? 1024 : 16], sm1[MX ? 1024 : 16];
    __shared__ int s_valid;
    const RingQ ring{{(lds_t*)sa0, (lds_t*)sa1}, {(lds_t*)sb0, (lds_t*)sb1}, s_tok, s_tscale, nullptr, s_wscale,
                     {(lds_t*)sm0, (lds_t*)sm1}};

    int blk, tg;
    if (!map_active_tile<true>(g, ngroups, blk, tg)) return;
    const int e = __builtin_amdgcn_readfirstlane(g.expert_ids[blk]);
    if (e < 0) return;
    const int tile0 = tg * ntw;
    const int R = g.T * g.topk;
    constexpr int K = NST * kKB;
    {
        constexpr int sbytes = MX ? K / 32 : (K / 128) * 4;   // activation scale bytes per row
        for (int r = threadIdx.x >> 2; r < kBM; r += kThreads / 4) {
            const int f = g.sorted_ids[blk * kBM + r];
            const int src = f < R ? blk * kBM + r : blk * kBM;   // padding rows read the block's first row
            if ((threadIdx.x & 3) == 0) s_tok[r] = uint32_t(src - blk * kBM) * uint32_t(K);
            const uint8_t* srcs = reinterpret_cast<const uint8_t*>(g.inter_scale) + size_t(src) * sbytes;
            for (int b = (threadIdx.x & 3) * 4; b < sbytes; b += 16)
                *reinterpret_cast<uint32_t*>(s_tscale + r * sbytes + b) = *reinterpret_cast<const uint32_t*>(srcs + b);
        }
    }
    if constexpr (!MX) {
        // [tile][128-row block][K stage] block scales of the workgroup's tiles
        const float* wsc = static_cast<const float*>(g.w2_scale);
        for (int idx = threadIdx.x; idx < ntw * 2 * NST; idx += kThreads) {
            const int c = idx / (2 * NST), rb = (idx / NST) & 1, kb = idx % NST;
            s_wscale[idx] = wsc[(size_t(e) * (g.H / 128) + size_t(tile0 + c) * 2 + rb) * NST + kb];
        }
    }
    if (threadIdx.x < 64) {
        int n = 0;
#pragma unroll
        for (int q = 0; q < kBM / 64; ++q) n += __popcll(__ballot(g.sorted_ids[blk * kBM + q * 64 + threadIdx.x] < R));
        if (threadIdx.x == 0) s_valid = n;
    }
    __syncthreads();
    const int live = (s_valid + 31) >> 5;
    const int grp = (threadIdx.x >> 6) >> 2;
    const int nu = grp == 1 ? min(live, 2) : max(0, min(live - 2, 2));
    switch (nu) {
        case 0: run_tiles_q2<MX, NST, 0>(g, ring, blk, tile0, ntw, e); break;
        case 1: run_tiles_q2<MX, NST, 1>(g, ring, blk, tile0, ntw, e); break;
        default: run_tiles_q2<MX, NST, 2>(g, ring, blk, tile0, ntw, e); break;
    }
}

template <typename Kern>
hipError_t launch(Kern kernel, const GemmArgs& g, int ntiles, hipStream_t s) {
    const int64_t n = int64_t(g.num_blocks) * ntiles;
    const int64_t grid = (n + 7) / 8 * 8;
    hipLaunchKernelGGL(kernel, dim3(unsigned(grid)), dim3(kThreads), 0, s, g, ntiles);
    return hipGetLastError();
}

// column tiles per workgroup of the short-K GEMM2 (a power of two dividing
// the tile count): 16 up to 64 routed rows per expert on average (one block
// per expert: the 256 experts' blocks of the fp8 layer make one round of
// workgroups), else 8.  Measured on the fp8 layer (E 256, H 4096, I 256; down
// GEMM us for 1 / 2 / 4 / 8 / 16 tiles): 1024 tokens 132 / 110 / 106 / 98 / 95,
// 2048 tokens 169 / 143 / 136 / 127 / 123, 8192 tokens 492 / 415 / 386 / 384 / 422.
int short_tiles_per_wg(int ntiles, int rows_per_expert) {
    int n = rows_per_expert <= 64 ? 16 : 8;
    while (n > 1 && ntiles % n != 0) n >>= 1;
    return n;
}

}  // namespace

bool gemm_large_q_supported(int H, int I) {
    return H % kTM == 0 && I % 128 == 0 && H % kKB == 0 && H <= kMaxK && I <= kMaxK;
}

int gemm_large_q_block_m() { return kBM; }

hipError_t launch_gemm1_large_q(const GemmArgs& g, bool mx, hipStream_t s) {
    if (g.block_m != kBM) return hipErrorInvalidValue;
    return mx ? launch(gemm_large_q_kernel<1, true>, g, g.I / 128, s)
              : launch(gemm_large_q_kernel<1, false>, g, g.I / 128, s);
}

hipError_t launch_gemm2_large_q(const GemmArgs& g, bool mx, hipStream_t s) {
    if (g.block_m != kBM) return hipErrorInvalidValue;
    if (g.I <= kShortK) {
        const int ntiles = g.H / kTM;
        const int ntw = short_tiles_per_wg(ntiles, g.T * g.topk / std::max(g.E, 1));
        const int ngroups = ntiles / ntw;
        const int64_t n = int64_t(g.num_blocks) * ngroups;
        const dim3 grid(unsigned((n + 7) / 8 * 8)), block(kThreads);
        void (*kern)(GemmArgs, int, int) =
            g.I == 2 * kKB ? (mx ? gemm2_large_q_short_kernel<true, 2> : gemm2_large_q_short_kernel<false, 2>)
                           : (mx ? gemm2_large_q_short_kernel<true, 1> : gemm2_large_q_short_kernel<false, 1>);
        hipLaunchKernelGGL(kern, grid, block, 0, s, g, ngroups, ntw);
        return hipGetLastError();
    }
    return mx ? launch(gemm_large_q_kernel<2, true>, g, g.H / kTM, s)
              : launch(gemm_large_q_kernel<2, false>, g, g.H / kTM, s);
}

}  // namespace moe
