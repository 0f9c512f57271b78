// LDS-tiled grouped GEMMs for many rows per expert (prefill), bf16.
//
// Same orientation as the weight-streaming path: the expert's weight rows are
// the MFMA M side, the block's tokens the N side (so the GEMM1 epilogue keeps a
// gate row and its up row in the same lane and register).  A workgroup of 8
// waves owns a 256-weight-row x 256-token tile of one expert block.  Wave w
// owns weight rows 64(w % 4) .. +63 and, with g = w / 4, the 32-token
// sub-tiles u with u % 2 == g, so the live sub-tiles of a block's partly
// filled tail split evenly between the two waves of a SIMD (waves w and w + 4
// share SIMD w % 4).
//
// K is walked in stages of 64 (128-byte rows, whole cache lines: from L2 a
// streaming probe moved 64-byte row pieces at 17-21 TB/s and 128-byte pieces
// at ~30 TB/s).  Operands move global -> LDS with direct-to-LDS loads
// (global_load_lds_dwordx4: lane i's 16 bytes land at the instruction's LDS
// address + 16 i; no staging registers) into two-slot rings, each slot a
// separate array so that the slot a load writes and the slot being read are
// told apart at compile time.  Group 0 (waves 0..3) loads the weight tile,
// group 1 (waves 4..7) the token tile: a wave's loads retire in order, and
// each group then waits only for its own.
//
// Each stage is multiplied in two halves of K = 32.  The two waves of a SIMD
// alternate between a memory phase (read a half's MFMA fragments from LDS
// into registers; at the first half also issue the next stage's loads) and a
// compute phase (16 MFMAs from those registers): group 1 starts one phase
// late, so at any time one wave of each SIMD multiplies while the other moves
// data.  Every phase ends in a workgroup barrier (s_barrier alone: the release
// fence of __syncthreads would wait for the loads in flight).  The next
// stage's loads go to the slot both groups finished reading in the previous
// stage; group 0 waits for its weight loads at the end of its last compute
// phase of the stage, group 1 for its token loads at the end of its last
// memory phase, each just before the barrier after which group 0 reads the
// next stage (3-4 phases after the loads were issued).
//
// LDS rows are 128 bytes (eight 16-byte chunks); chunk c of row r sits at
// position c ^ ((r >> 1) & 7), which spreads the rows a fragment read touches
// over all banks.  The loads apply the same swizzle on the global side (lane
// i of a load fetches the chunk that belongs at its LDS position).
//
// MFMA v_mfma_f32_32x32x16_bf16 (layout checked on gfx950): lane l holds row
// (l % 32) of A / column (l % 32) of B at K offset (l / 32) * 8; the 32x32
// result gives lane l column (l % 32) and rows (i / 4) * 8 + (l / 32) * 4 + i % 4.
//
// Token sub-tiles that hold only padding (the tail of an expert's last block)
// are neither multiplied nor stored: the loop is instantiated per wave for
// 0..4 live sub-tiles.  An expert's last block with at most 64 real rows is
// taken by the workgroup of the expert's previous (full) block as token rows
// 256..319 (sub-tiles 8 and 9, so 4 or 5 per wave): the expert's weight tiles
// stream once for both blocks.  With routing near 256 rows per expert about
// half of the experts end in such a block, which otherwise re-streams every
// weight tile for a few rows.  Padding rows load a real row of the block (they
// are never stored), which L2 holds.
//
//   GEMM1 (a4+a5): tile = 128 intermediate columns: gate rows c0..c0+127 and
//                  up rows I+c0..; wave w owns gate rows c0+32(w%4).. and the
//                  matching up rows; epilogue a = bf16(bf16(silu(bf16 g)) *
//                  bf16 u) stored in expert-sorted order (P2 sections 1.1, 1.2).
//   GEMM2 (a6):    tile = 256 output columns h; wave w owns h0+64(w%4)..;
//                  epilogue y[f] = tw[f] * acc in fp32 (P2 section 1.1).
//   The layer variants (router weight on the input, SwiGLU clamp) act in the
//   epilogues as in the weight-streaming kernels.
#include "common.h"

namespace moe {

namespace {

constexpr int kTM = 256;           // weight rows per workgroup
constexpr int kBM = 256;           // tokens per workgroup (= block_m of the alignment)
constexpr int kKB = 64;            // K per stage (bf16 elements)
constexpr int kRowBytes = kKB * 2; // 128 bytes per LDS row
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kXR = 64;            // rows a workgroup may take from the expert's next block
constexpr int kBR = kBM + kXR;     // token rows of the LDS token tile
constexpr int kSlotA = kTM * kRowBytes;   // 32 KiB
constexpr int kSlotB = kBR * kRowBytes;   // 40 KiB
constexpr int kLoadRows = 1024 / kRowBytes;   // rows one direct-to-LDS load fills (64 lanes x 16 bytes)
constexpr int kLoads = kTM / 4 / kLoadRows;   // loads per wave per stage (4 waves per tile)
static_assert(kTM == kBM, "both groups load 64 rows per wave");
static_assert(kXR == 4 * 2 * kLoadRows, "each group-1 wave loads 16 extension rows in two loads");
static_assert(2 * (kSlotA + kSlotB) + kBR * 4 + 4 <= 160 * 1024, "the rings fit the LDS");

typedef __attribute__((address_space(3))) uint8_t lds_t;

__device__ __forceinline__ uint32_t swz_chunk(int row, int chunk) { return uint32_t(chunk ^ ((row >> 1) & 7)) << 4; }

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14)
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

struct Ring {
    lds_t* a[2];
    lds_t* b[2];
    const uint32_t* tok;   // byte offset of each token-tile row's source row (LDS table)
};

template <int GEMM, int NU, bool kExt>
__device__ __forceinline__ void run_tile(const GemmArgs& g, const Ring& ring, int blk, int tile, int e) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv & 3, grp = wv >> 2;
    const int K = GEMM == 1 ? g.H : g.I;
    const int nst = K / kKB;
    const uint32_t kbytes = uint32_t(K) * 2;

    // ---- load sources.  Load q of a wave fills LDS rows 64 lw + 8 q + i/8
    //      (lane i), position i % 8, with the global chunk that belongs there:
    //      (i % 8) ^ ((row >> 1) & 7) = (i % 8) ^ ((i / 16 + 4 q) % 8).  ---------
    const int lw = wm;                        // index inside the load group
    const int lrow = lane >> 3;
    const uint32_t lchunk_even = uint32_t((lane & 7) ^ ((lane >> 4) & 7)) << 4;
    const uint32_t lchunk_odd = uint32_t((lane & 7) ^ (((lane >> 4) + 4) & 7)) << 4;
    const uint8_t* abase;
    const uint8_t* bbase;
    if constexpr (GEMM == 1) {
        abase = static_cast<const uint8_t*>(g.w13) + size_t(e) * 2 * g.I * kbytes;
        bbase = reinterpret_cast<const uint8_t*>(g.x);
    } else {
        abase = static_cast<const uint8_t*>(g.w2) + (size_t(e) * g.H + size_t(tile) * kTM) * kbytes;
        bbase = static_cast<const uint8_t*>(g.inter) + size_t(blk) * kBM * kbytes;
    }
    // weight rows of load q: wave lw's 64 tile rows are 32 gate rows then the
    // 32 matching up rows (GEMM1), or 64 consecutive rows of W2's tile (GEMM2)
    auto weight_row0 = [&](int q) -> size_t {
        if constexpr (GEMM == 1) return size_t(q >= 4 ? g.I : 0) + tile * 128 + lw * 32 + 8 * (q & 3);
        else return size_t(64 * lw + 8 * q);
    };
    const uint32_t a_lane = uint32_t(lrow) * kbytes;

    // the K walk starts at a stage that depends on (expert, tile), so that the
    // workgroups do not all read the same offset of their 2^k-byte rows at once
    // (a streaming probe of the weight loads alone: 5.2 -> 6.2 TB/s).  The
    // column tiles of one block, which share its token rows, start one stage
    // apart: they then read each token line within a few stages of each other,
    // which L2 holds, without all asking for the same lines at the same time.
    // Prefill layer (GEMM1 / GEMM2 ms, HBM read bytes of GEMM1): no rotation
    // 1.137 / 0.688, 3.58 GB; start keyed by expert only 1.11 / 0.68, 3.59 GB;
    // by (expert, 13 x tile) 1.10 / 0.635, 5.0 GB; by (expert, tile) 1.068 /
    // 0.623, 3.62 GB.  It depends on (expert, tile) only, so every output
    // keeps one K order.
    const int rot = (e * 7 + tile) % nst;
    auto kofs = [&](int st) -> uint32_t {
        const int k = st + rot;
        return uint32_t(k < nst ? k : k - nst) * kRowBytes;
    };
    auto issue_a = [&](int st, lds_t* A) {   // group 0: 64 weight rows per wave
        const uint8_t* base = abase + kofs(st);
#pragma unroll
        for (int q = 0; q < kLoads; ++q)
            load_lds(base + weight_row0(q) * kbytes, a_lane + ((q & 1) ? lchunk_odd : lchunk_even),
                     A + (64 * lw + kLoadRows * q) * kRowBytes);
    };
    auto issue_b = [&](int st, lds_t* B) {   // group 1: 64 token rows per wave (+ 16 extension rows)
        const uint8_t* base = bbase + kofs(st);
#pragma unroll
        for (int q = 0; q < kLoads; ++q) {
            const int row = 64 * lw + kLoadRows * q + lrow;
            load_lds(base, ring.tok[row] + ((q & 1) ? lchunk_odd : lchunk_even), B + (row - lrow) * kRowBytes);
        }
        if constexpr (kExt) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int row = kBM + 16 * lw + kLoadRows * q + lrow;
                load_lds(base, ring.tok[row] + ((q & 1) ? lchunk_odd : lchunk_even), B + (row - lrow) * kRowBytes);
            }
        }
    };

    // ---- fragment addresses: rows 64 wm + fr (+32 for the up rows) and
    //      32 grp + fr (+64 per sub-tile pair); K16 step t of a stage reads
    //      chunk 2t + fk, swizzled by the row (the same for all these rows) ----
    const int fr = lane & 31;   // fragment row / column
    const int fk = lane >> 5;   // fragment K half
    uint32_t coff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) coff[t] = swz_chunk(fr, 2 * t + fk);
    const uint32_t a_row = uint32_t(64 * wm + fr) * kRowBytes;
    const uint32_t b_row = uint32_t(32 * grp + fr) * kRowBytes;

    f32x16 acc[2][NU > 0 ? NU : 1];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int u = 0; u < (NU > 0 ? NU : 1); ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][u][i] = 0.0f;
    i32x4 af[2][2], bfr[NU > 0 ? NU : 1][2];

    typedef const __attribute__((address_space(3))) i32x4 lds_v4;
    auto read_half = [&](const lds_t* A, const lds_t* B, int h) {
        if constexpr (NU > 0) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t c = coff[2 * h + j];
#pragma unroll
                for (int a = 0; a < 2; ++a) af[a][j] = *reinterpret_cast<lds_v4*>(A + a_row + c + a * 32 * kRowBytes);
#pragma unroll
                for (int u = 0; u < NU; ++u) bfr[u][j] = *reinterpret_cast<lds_v4*>(B + b_row + c + u * 64 * kRowBytes);
            }
        }
    };
    auto compute = [&]() {
        if constexpr (NU > 0) {
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int u = 0; u < NU; ++u)
#pragma unroll
                    for (int a = 0; a < 2; ++a)
                        acc[a][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[a][j]),
                                                                            __builtin_bit_cast(bf16x8, bfr[u][j]),
                                                                            acc[a][u], 0, 0, 0);
            __builtin_amdgcn_s_setprio(0);
        }
    };
    // one stage: slots (A, B) hold it, (An, Bn) receive the next one
    auto stage = [&](int s, const lds_t* A, const lds_t* B, lds_t* An, lds_t* Bn) {
        const bool more = s + 1 < nst;
        // memory phase, first half: fragments, then the next stage's loads
        read_half(A, B, 0);
        if (more) {
            if (grp == 0) issue_a(s + 1, An);
            else issue_b(s + 1, Bn);
        }
        wait_lgkm0();
        barrier();
        compute();
        barrier();
        // memory phase, second half (group 1: its token loads must have landed)
        read_half(A, B, 1);
        wait_lgkm0();
        if (grp == 1) wait_vm0();
        barrier();
        compute();
        if (grp == 0) wait_vm0();   // its weight loads of the next stage
        barrier();
    };

    // ---- prologue: stage 0 in LDS ----------------------------------------------
    if (grp == 0) issue_a(0, ring.a[0]);
    else issue_b(0, ring.b[0]);
    wait_vm0();
    barrier();
    if (grp == 1) barrier();   // group 1 runs one phase behind group 0

    for (int s = 0; s < nst; s += 2) {
        stage(s, ring.a[0], ring.b[0], ring.a[1], ring.b[1]);
        if (s + 1 < nst) stage(s + 1, ring.a[1], ring.b[1], ring.a[0], ring.b[0]);
    }
    if (grp == 0) barrier();   // the barrier group 1 ran at the start

    // ---- epilogues: wave sub-tile u sits at token rows (2u + grp) * 32 ---------
    const int R = g.T * g.topk;
    if constexpr (GEMM == 1) {
        uint16_t* out = static_cast<uint16_t*>(g.inter);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int row = blk * kBM + (2 * u + grp) * 32 + fr;
            const float w_in = gemm1_row_weight(g, g.sorted_ids[row]);
            const int colw = tile * 128 + wm * 32;
#pragma unroll
            for (int q = 0; q < 4; ++q) {   // groups of 4 consecutive columns
                uint32_t p[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int i0 = q * 4 + 2 * h;
                    const float a0 = swiglu_bf16(acc[0][u][i0], acc[1][u][i0], w_in, g.clamp, g.clamp_limit);
                    const float a1 = swiglu_bf16(acc[0][u][i0 + 1], acc[1][u][i0 + 1], w_in, g.clamp, g.clamp_limit);
                    p[h] = uint32_t(f32_to_bf16_rne(a0)) | (uint32_t(f32_to_bf16_rne(a1)) << 16);
                }
                const int col = colw + q * 8 + fk * 4;
                *reinterpret_cast<i32x2*>(out + int64_t(row) * g.I + col) = i32x2{int(p[0]), int(p[1])};
            }
        }
    } else {
        const int hw = tile * kTM + wm * 64;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int f = g.sorted_ids[blk * kBM + (2 * u + grp) * 32 + fr];
            if (f >= R) continue;
            const float tw = gemm2_row_weight(g, f);
            float* yrow = g.y + int64_t(f) * g.H;
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f32x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = __fmul_rn(acc[a][u][q * 4 + j], tw);
                    *reinterpret_cast<f32x4*>(yrow + hw + a * 32 + q * 8 + fk * 4) = v;
                }
        }
    }
}

template <int GEMM>
__global__ __launch_bounds__(kThreads, 1) void gemm_large_kernel(GemmArgs g, int ntiles) {
    __shared__ __attribute__((aligned(1024))) uint8_t sa0[kSlotA], sa1[kSlotA];
    __shared__ __attribute__((aligned(1024))) uint8_t sb0[kSlotB], sb1[kSlotB];
    __shared__ uint32_t s_tok[kBR];
    __shared__ int s_valid;
    const Ring ring{{(lds_t*)sa0, (lds_t*)sa1}, {(lds_t*)sb0, (lds_t*)sb1}, s_tok};

    int blk, tile;
    // block-major: the 12-24 column tiles of one block share its token rows in
    // L2, and the blocks of one expert (adjacent) run together and share the
    // weight tiles
    if (!map_active_tile<true>(g, ntiles, blk, tile)) return;
    const int e = __builtin_amdgcn_readfirstlane(g.expert_ids[blk]);
    if (e < 0) return;
    {
        // An expert with three or more blocks (the hot experts of a skewed
        // routing) takes its items column tile first, then block: its blocks
        // then read each weight tile at about the same time and share it in
        // L2 instead of re-streaming all its weights once per block (skewed
        // layer at 8192 tokens: GEMM1 fetched 19.9 GB for 13.5 GB of
        // weights).  Experts with one or two blocks keep the block-major
        // order, whose column tiles share the block's token rows in L2 (the
        // tile-first order for them too cost prefill 1.86 -> 2.11 ms).  A
        // permutation of the expert's own items: every output is the same.
        const int act = __builtin_amdgcn_readfirstlane(g.ntpp[0]) / kBM;
        int first = blk, last = blk;
        while (first > 0 && g.expert_ids[first - 1] == e) --first;
        while (last + 1 < act && g.expert_ids[last + 1] == e) ++last;
        const int nb = last - first + 1;
        if (nb >= 3) {
            const int li = (blk - first) * ntiles + tile;
            tile = li / nb;
            blk = first + li % nb;
        }
    }

    // An expert's last block with at most kXR real rows (row kXR is padding)
    // rides along with the expert's previous block: that workgroup multiplies
    // its rows as token rows 256..319 of the same weight tiles, so the expert's
    // weights stream once for both (each output keeps its K order: results are
    // the same bits).
    const int R = g.T * g.topk;
    const int active = __builtin_amdgcn_readfirstlane(g.ntpp[0]) / kBM;
    auto short_tail = [&](int b) { return g.sorted_ids[b * kBM + kXR] >= R; };
    if (blk > 0 && g.expert_ids[blk - 1] == e && short_tail(blk)) return;
    const bool ext = blk + 1 < active && g.expert_ids[blk + 1] == e && short_tail(blk + 1);

    // the token tile's source rows (padding rows read a real row of the block,
    // never stored), and the count of rows that hold real slots (a prefix)
    {
        const uint32_t kb = uint32_t(GEMM == 1 ? g.H : g.I) * 2;
        const int first = g.sorted_ids[blk * kBM];
        for (int r = threadIdx.x; r < kBR; r += kThreads) {
            const int f = (r < kBM || ext) ? g.sorted_ids[blk * kBM + r] : R;
            if (GEMM == 1) s_tok[r] = uint32_t((f < R ? f : first) / g.topk) * kb;
            else s_tok[r] = uint32_t(f < R ? r : 0) * kb;
        }
    }
    if (threadIdx.x < 64) {
        int n = 0;
#pragma unroll
        for (int q = 0; q < kBR / 64; ++q)
            if (q < kBM / 64 || ext) n += __popcll(__ballot(g.sorted_ids[blk * kBM + q * 64 + threadIdx.x] < R));
        if (threadIdx.x == 0) s_valid = n;
    }
    __syncthreads();
    const int valid = s_valid;
    // live 32-token sub-tiles of this wave: u = grp, grp + 2, ... below the count
    const int live = (valid + 31) >> 5;
    const int grp = (threadIdx.x >> 6) >> 2;
    const int nu = (live - grp + 1) >> 1;
    if (ext) {   // 257..320 rows: 4 or 5 sub-tiles per wave
        if (nu >= 5) run_tile<GEMM, 5, true>(g, ring, blk, tile, e);
        else run_tile<GEMM, 4, true>(g, ring, blk, tile, e);
        return;
    }
    switch (nu) {
        case 0: run_tile<GEMM, 0, false>(g, ring, blk, tile, e); break;
        case 1: run_tile<GEMM, 1, false>(g, ring, blk, tile, e); break;
        case 2: run_tile<GEMM, 2, false>(g, ring, blk, tile, e); break;
        case 3: run_tile<GEMM, 3, false>(g, ring, blk, tile, e); break;
        default: run_tile<GEMM, 4, false>(g, ring, blk, tile, e); break;
    }
}

template <typename Kern>
hipError_t launch(Kern kernel, const GemmArgs& g, int ntiles, hipStream_t s) {
    const int64_t n = int64_t(g.num_blocks) * ntiles;
    const int64_t grid = (n + 7) / 8 * 8;
    hipLaunchKernelGGL(kernel, dim3(unsigned(grid)), dim3(kThreads), 0, s, g, ntiles);
    return hipGetLastError();
}

}  // namespace

bool gemm_large_supported(int H, int I, bool fp8) {
    return !fp8 && I % 128 == 0 && H % kTM == 0 && H % kKB == 0 && I % kKB == 0;
}

int gemm_large_block_m() { return kBM; }

hipError_t launch_gemm1_large(const GemmArgs& g, bool fp8, hipStream_t s) {
    if (fp8 || g.block_m != kBM) return hipErrorInvalidValue;
    return launch(gemm_large_kernel<1>, g, g.I / 128, s);
}

hipError_t launch_gemm2_large(const GemmArgs& g, bool fp8, hipStream_t s) {
    if (fp8 || g.block_m != kBM) return hipErrorInvalidValue;
    return launch(gemm_large_kernel<2>, g, g.H / kTM, s);
}

}  // namespace moe
