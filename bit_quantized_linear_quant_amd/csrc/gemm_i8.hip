// int8 x int8 -> int32 tiled GEMM on gfx950 matrix cores, with the dequant
// epilogue fused ("Per-token Quantization for Matmul": Input, Output and
// Example; "Q4LinearFunction" forward for the per-tensor scale pair).
//
// The int8 kernels share the epilogue:
//
// gemm_i8_big_kernel -- large products with [n][k] weights and k % 64 == 0
//   whose 256 x 256 tiles number at least 128 per launch (the 8192^3 A4W4
//   product; fewer tiles leave compute units idle and the 128 x 128 kernel
//   below is faster).  A 512-thread workgroup owns a 256 x 256
//   output tile, each of its eight waves (two per SIMD) a 128 x 64 part
//   held as 4 x 2 blocks of v_mfma_i32_32x32x32_i8; the two groups of four
//   waves run opposite phases of every slice (fragment reads and loads
//   against products).  64-byte k-slices of A and B move from HBM straight
//   into LDS with global_load_lds_dwordx4 (no register staging) through a
//   ring of three slices, so two slices stream in while the matrix cores
//   consume the third; explicit vmcnt waits and two barriers per slice.  In LDS each
//   16-byte chunk c of row r sits at chunk position c ^ swz(r), which puts
//   the 16 rows read together by a fragment load in distinct bank groups.
//   Tiles are ordered so that each XCD (workgroup id mod 8) walks its own
//   band of tile rows, four rows at a time, so concurrently running tiles
//   share A and B slices in that XCD's L2.  Rows past m or n are loaded
//   clamped and never stored.  16-bit outputs leave through a padded LDS
//   tile as whole row segments.
//
// gemv_i8_kernel -- decode shapes: m <= 64 (or m <= 128 with at most 6144
//   columns) with [n][k] weights and k % 64 == 0.  The token rows fill up
//   to eight 16-row matrix-core blocks;
//   waves split k over a few 16-column blocks per workgroup, reading the
//   weights once with streaming loads, and sum their partials in LDS.
//
// gemv_kn_i8_kernel -- the same shapes with [k][n] weights (m <= 64,
//   k % 64 == 0, n % 4 == 0): 4 x 4 byte blocks of the weight rows are
//   transposed in registers and turned into fragments through a per-wave
//   LDS block.
//
// gemm_i8_kernel -- everything else (any m, n, k >= 1, weights [k][n] or
//   [n][k]): 128 x 128 tiles, 2 x 2 waves of 64 x 64 in 32x32x32 MFMA blocks,
//   register-staged loads with zero fill at the edges, LDS rows padded to
//   80 bytes; [k][n] weights are transposed 4 x 4 bytes at a time in
//   registers on their way into LDS.
//
// The 4-bit A4W4 products of the same file run on the FP6 matrix cores
// (gemm_a4w4_f6_kernel on FP6 operand tiles, gemm_a4w4_packed_kernel on
// operands of two 4-bit codes per byte) with the large-tile epilogue.
#include "ql_device.hpp"
#include "ql_launch.hpp"
#include "gemm_ring.hpp"

#include <type_traits>

namespace ql {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

struct Params {
    const int8_t *x;
    const int8_t *w;
    const float *pts;
    const float *deq;
    const float *sa;
    const float *sw;
    float eps;
    int64_t m, n, k;
    void *out;
    const float *bias;   // [n] or NULL
    // element strides between batches (blockIdx.z); out's in bytes
    int64_t bx, bw, bpts, bdeq, bout;
};

// Move the operand pointers to this workgroup's batch (grid z).  A
// non-batched launch has one z and leaves them as they are.
__device__ __forceinline__ void to_batch(Params &p) {
    const int64_t b = blockIdx.z;
    p.x += b * p.bx;
    p.w += b * p.bw;
    if (p.pts) p.pts += b * p.bpts;
    if (p.deq) p.deq += b * p.bdeq;
    p.out = static_cast<char *>(p.out) + b * p.bout;
}

// Per-row and per-column epilogue factors: (acc * row) * col, rounded once
// per multiply in fp32, then to the output type.  Per-row factors of a tile
// are staged in LDS and per-column factors loaded before the store loops, so
// no output element waits on a global load of its own.
template <int EPI, int OUT>
struct Epilogue {
    float sa = 0.f, sw = 0.f;
    const float *rowf = nullptr;  // LDS copy of the tile's per-row factors
    __device__ __forceinline__ void init(const Params &p) {
        if (EPI == EPI_SCALARS && OUT != OUT_I32) {
            const float a = *p.sa, w = *p.sw;
            sa = a > p.eps ? a : p.eps;
            sw = w > p.eps ? w : p.eps;
        }
    }
    // Called by every thread of the workgroup, after the last read of `lds`
    // by the main loop; a barrier must follow before row_factor is used.
    __device__ __forceinline__ void stage_rows(const Params &p, int64_t m0, int rows, float *lds) {
        if (EPI == EPI_ROWCOL && OUT != OUT_I32) {
            for (int r = threadIdx.x; r < rows; r += blockDim.x) lds[r] = p.pts[m0 + r < p.m ? m0 + r : p.m - 1];
            rowf = lds;
        }
    }
    __device__ __forceinline__ float col_factor(const Params &p, int64_t col) const {
        if (OUT == OUT_I32) return 0.f;
        return EPI == EPI_ROWCOL ? p.deq[col < p.n ? col : p.n - 1] : sw;
    }
    // `local` is the row's index within the staged tile.
    __device__ __forceinline__ float row_factor(int local) const {
        if (OUT == OUT_I32) return 0.f;
        return EPI == EPI_ROWCOL ? rowf[local] : sa;
    }
    // bias of a column (0 when there is none; value() adds it only if p.bias)
    __device__ __forceinline__ float col_bias(const Params &p, int64_t col) const {
        return (OUT == OUT_I32 || !p.bias) ? 0.f : p.bias[col < p.n ? col : p.n - 1];
    }
    // fl32(fl32(acc * row) * col), then + bias in fp32
    __device__ __forceinline__ float value(const Params &p, int32_t v, float rf, float cf, float cb) const {
        const float y = __fmul_rn(__fmul_rn((float)v, rf), cf);
        return p.bias ? __fadd_rn(y, cb) : y;
    }
    __device__ __forceinline__ void store(const Params &p, int64_t row, int64_t col, int32_t v, float rf,
                                          float cf, float cb) const {
        const int64_t idx = row * p.n + col;
        if (OUT == OUT_I32) static_cast<int32_t *>(p.out)[idx] = v;
        else store_out<OUT>(p.out, idx, value(p, v, rf, cf, cb));
    }
};

// ---------------------------------------------------------------------------
// Large-tile kernel
// ---------------------------------------------------------------------------
// Epilogue of the 256 x 256 tile kernels: lane holds column lane%32 of each
// 32x32 block and rows 8*(r/4) + 4*(lane/32) + r%4 of register r.  The
// accumulators are int32, or fp32 holding integers below 2^24 (exact).
__device__ __forceinline__ int32_t acc_i32(int32_t v) { return v; }
__device__ __forceinline__ int32_t acc_i32(float v) { return (int32_t)v; }

// The wave's sub-tile is 128 rows (wm) x 32 BJ columns (wn); LDS needs
// 1024 + waves x 128 x big_epitch(BJ) bytes.
constexpr int big_epitch(int bj) { return 64 * bj + 16; }

template <int EPI, int OUT, int BJ, typename ACC>
__device__ __forceinline__ void big_epilogue(const Params &p, const ACC (&acc)[4][BJ], int8_t *smem, int64_t m0,
                                             int64_t n0, int wm, int wn, int wave, int lane) {
    constexpr int EPITCH = big_epitch(BJ);
    constexpr int PIECES = 4 * BJ;        // 16-byte pieces of a sub-tile row
    constexpr int RPQ = kWave / PIECES;   // rows per store instruction
    const int fr = lane % 32;
    const int64_t c0 = n0 + wn * 32 * BJ;
    Epilogue<EPI, OUT> ep;
    ep.init(p);
    ep.stage_rows(p, m0, LB, reinterpret_cast<float *>(smem));
    __syncthreads();
    float cf[BJ], cb[BJ];
#pragma unroll
    for (int j = 0; j < BJ; j++) {
        cf[j] = ep.col_factor(p, c0 + 32 * j + fr);
        cb[j] = ep.col_bias(p, c0 + 32 * j + fr);
    }
    if constexpr (OUT == OUT_F16 || OUT == OUT_BF16) {
        // Through LDS: the wave rounds its sub-tile into a padded LDS tile
        // (the two row groups of one write land 16 banks apart), then writes
        // whole row segments, 16 bytes per lane.
        int8_t *tile = smem + 1024 + wave * 128 * EPITCH;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int lr = 32 * i + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                const float rf = ep.row_factor(wm * 128 + lr);
#pragma unroll
                for (int j = 0; j < BJ; j++) {
                    const float y = ep.value(p, acc_i32(acc[i][j][r]), rf, cf[j], cb[j]);
                    *reinterpret_cast<uint16_t *>(tile + lr * EPITCH + 2 * (32 * j + fr)) =
                        OUT == OUT_F16 ? f32_to_f16_rne(y) : f32_to_bf16_rne(y);
                }
            }
        // each wave reads back only its own sub-tile
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < 128 / RPQ; q++) {
            const int lr = RPQ * q + lane / PIECES, piece = lane % PIECES;
            const uint4 v = *reinterpret_cast<const uint4 *>(tile + lr * EPITCH + 16 * piece);
            const int64_t row = m0 + wm * 128 + lr, col = c0 + 8 * piece;
            if (row < p.m) {
                uint16_t *dst = static_cast<uint16_t *>(p.out) + row * p.n + col;
                if (col + 8 <= p.n && (p.n % 8) == 0) {
                    *reinterpret_cast<uint4 *>(dst) = v;
                } else {
                    const uint16_t h[8] = {(uint16_t)v.x, (uint16_t)(v.x >> 16), (uint16_t)v.y, (uint16_t)(v.y >> 16),
                                           (uint16_t)v.z, (uint16_t)(v.z >> 16), (uint16_t)v.w, (uint16_t)(v.w >> 16)};
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        if (col + e < p.n) dst[e] = h[e];
                }
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < BJ; j++) {
        const int64_t col = c0 + 32 * j + fr;
        if (col >= p.n) continue;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int local = wm * 128 + 32 * i + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                if (m0 + local < p.m) ep.store(p, m0 + local, col, acc_i32(acc[i][j][r]), ep.row_factor(local), cf[j], cb[j]);
            }
    }
}

template <int BK, int NBUF, int EPI, int OUT>
__global__ __launch_bounds__(2 * LThreads, 1) void gemm_i8_big_kernel(Params p, int tiles_m, int tiles_n) {
    constexpr int STAGE = 2 * BigTile<BK>::TILE;
    // main loop: a ring of NBUF (A, B) slices; epilogue: 1 KB of row factors,
    // then one padded 128 x 64 output sub-tile per wave (2-byte outputs)
    constexpr int EPI_BYTES = 1024 + 8 * 128 * big_epitch(2);
    constexpr int SMEM = NBUF * STAGE > EPI_BYTES ? NBUF * STAGE : EPI_BYTES;
    __shared__ __attribute__((aligned(1024))) int8_t smem[SMEM];

    to_batch(p);
    const int lane = threadIdx.x % kWave, wave = wave_id();
    const int wm = wave % 2, wn = (wave / 2) % 4;
    int tm, tn;
    xcd_tile(blockIdx.x, tiles_m, tiles_n, kGroupM, tm, tn);
    const int64_t m0 = (int64_t)tm * LB, n0 = (int64_t)tn * LB;
    v16i acc[4][2];
    ring_gemm_pp<BK, NBUF, MK_I8>(acc, smem, p.x, p.w, p.m, p.n, p.k, m0, n0, wm, wn, lane, wave);
    big_epilogue<EPI, OUT>(p, acc, smem, m0, n0, wm, wn, wave, lane);
}

// ---------------------------------------------------------------------------
// 4-bit product on FP6 E3M2 operand tiles
// ---------------------------------------------------------------------------
// The 256 x 256 tile of the large-tile kernel on
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E3M2 and unit block
// scales: twice the int8 matrix-core rate per instruction.  Codes are
// integers in [-8, 7], so every product and partial sum is an integer of
// magnitude at most 64 k < 2^23 (k <= 131071): the fp32 accumulation is
// exact and equals the int32 one.  Operand tiles (quant_a4w4_tiles_kernel):
// 32 rows x 64 k in 1536 bytes, lane l's register image at 16l (16 bytes)
// and 1024 + 8l (8 bytes); a 128-k slice of a 32-row block is two adjacent
// tiles, so slices copy to LDS unchanged and every fragment is one 16-byte
// and one 8-byte read by consecutive lanes.
//
// Eight waves, two per SIMD (waves w and w + 4 share SIMD w % 4), each own a
// 128 x 64 sub-tile (4 x 2 blocks of 32 x 32).  The two groups of four
// waves run opposite phases of a slice: while one group issues its 16
// products, its SIMD partners read their fragments of the slice from LDS
// and issue their share of the direct global -> LDS loads two slices ahead,
// so the matrix cores see a ready wave at every phase.  Two workgroup
// barriers per slice separate the phases; the second group passes one extra
// barrier at the start and the first group one at the end, which puts them
// half a slice apart.  Before every barrier a wave waits until at most one
// slice of its own loads is in flight, so a slice has fully landed (all
// waves' loads) at the barrier before the first read of it, and a ring of
// three LDS slices is never overwritten while a partner still reads it.
constexpr int kF6Tile = 1536;
constexpr int kF6Op = 8 * 2 * kF6Tile;        // one operand's 256-row x 128-k slice
constexpr int kF6Buf = 3;                     // LDS slices in the ring
constexpr int kF6Waves = 8;
constexpr int kF6Loads = kF6Op / 1024 / kF6Waves;   // 1 KB direct loads per wave and operand
constexpr int kF6Scale = 0x7f7f7f7f;          // E8M0 127 (2^0) in every byte

__device__ __forceinline__ v8i f6_frag(const int8_t *tile, int lane) {
    const uint4 a = *reinterpret_cast<const uint4 *>(tile + 16 * lane);
    const uint2 b = *reinterpret_cast<const uint2 *>(tile + 1024 + 8 * lane);
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, 0, 0};
}

template <int OUT>
__global__ __launch_bounds__(kF6Waves * kWave, 1) void gemm_a4w4_f6_kernel(Params p, int tiles_m, int tiles_n) {
    constexpr int STAGE = 2 * kF6Op;
    constexpr int EPI_BYTES = 1024 + kF6Waves * 128 * big_epitch(2);
    constexpr int SMEM = kF6Buf * STAGE > EPI_BYTES ? kF6Buf * STAGE : EPI_BYTES;
    __shared__ __attribute__((aligned(1024))) int8_t smem[SMEM];

    const int lane = threadIdx.x % kWave, wave = wave_id();
    const int group = wave / 4;
    const int wm = wave % 2, wn = (wave / 2) % 4;   // 2 x 4 sub-tiles of 128 x 64
    int tm, tn;
    xcd_tile(blockIdx.x, tiles_m, tiles_n, kGroupM, tm, tn);
    const int64_t m0 = (int64_t)tm * LB, n0 = (int64_t)tn * LB;
    const int64_t ktiles = (p.k + 127) / 128 * 2;   // 64-k tiles per 32-row block
    const int64_t nk = ktiles / 2;                   // 128-k slices
    const int64_t rows_a = (p.m + 31) / 32, rows_b = (p.n + 31) / 32;

    // Direct load `inst` of a slice copies 1 KB: 32-row block inst / 3 of
    // the tile, piece inst % 3 of its two adjacent 64-k tiles.  Blocks past
    // the operand re-read its last block; those rows are never stored.
    const int8_t *srcA[kF6Loads];
    const int8_t *srcB[kF6Loads];
#pragma unroll
    for (int ii = 0; ii < kF6Loads; ii++) {
        const int inst = wave * kF6Loads + ii;
        const int rt = inst / 3, piece = inst % 3;
        const int64_t ra = min(m0 / 32 + rt, rows_a - 1), rb = min(n0 / 32 + rt, rows_b - 1);
        srcA[ii] = p.x + ra * ktiles * kF6Tile + 1024 * piece + 16 * lane;
        srcB[ii] = p.w + rb * ktiles * kF6Tile + 1024 * piece + 16 * lane;
    }
    // slices past the end re-read the last one into the ring's free slot
    auto issue = [&](int64_t slice, int buf) __attribute__((always_inline)) {
        const int64_t off = (slice < nk ? slice : nk - 1) * 2 * kF6Tile;
#pragma unroll
        for (int ii = 0; ii < kF6Loads; ii++) {
            const int inst = wave * kF6Loads + ii;
            lds_load16(srcA[ii] + off, smem + buf * STAGE + 1024 * inst);
            lds_load16(srcB[ii] + off, smem + buf * STAGE + kF6Op + 1024 * inst);
        }
    };

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = v16f{};

    issue(0, 0);
    issue(1, 1);
    if (group == 1) {
        wait_vmcnt<2 * kF6Loads>();
        barrier_only();
    }
    for (int64_t kt = 0; kt < nk; kt++) {
        // fragment phase: this slice to registers, slice kt + 2 requested
        wait_vmcnt<2 * kF6Loads>();
        barrier_only();
        const int8_t *cur = smem + (int)(kt % kF6Buf) * STAGE;
        v8i fa[2][4], fb[2][2];
#pragma unroll
        for (int st = 0; st < 2; st++) {
#pragma unroll
            for (int i = 0; i < 4; i++) fa[st][i] = f6_frag(cur + ((wm * 4 + i) * 2 + st) * kF6Tile, lane);
#pragma unroll
            for (int j = 0; j < 2; j++) fb[st][j] = f6_frag(cur + kF6Op + ((wn * 2 + j) * 2 + st) * kF6Tile, lane);
        }
        issue(kt + 2, (int)((kt + 2) % kF6Buf));
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the fragments are in registers
        wait_vmcnt<2 * kF6Loads>();
        barrier_only();
        // product phase
#pragma unroll
        for (int st = 0; st < 2; st++)
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[st][i], fb[st][j], acc[i][j], 3, 3,
                                                                                0, kF6Scale, 0, kF6Scale);
    }
    if (group == 0) barrier_only();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    big_epilogue<EPI_SCALARS, OUT>(p, acc, smem, m0, n0, wm, wn, wave, lane);
}

template <int OUT>
hipError_t launch_f6(const Params &p, hipStream_t st) {
    const int64_t tm = (p.m + LB - 1) / LB, tn = (p.n + LB - 1) / LB;
    if (tm * tn > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_a4w4_f6_kernel<OUT>), dim3((unsigned)(tm * tn)), dim3(kF6Waves * kWave), 0, st, p,
                       (int)tm, (int)tn);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 4-bit product on packed two-per-byte operands
// ---------------------------------------------------------------------------
// The operands hold 0.5 byte per code (quant_a4w4_packed_kernel) on the FP6
// operand's tile grid: a 1024-byte tile per 32 rows x 64 k, slot l (16
// bytes) holding the 32 codes of lane l's register image.  The 16 KB of each
// operand that a 128-k slice of the 256 x 256 tile needs move HBM ->
// registers, one slot (16 bytes) per load, two slices ahead in two register
// sets; each slot becomes 32 exact fp16 values (code + 8 ORed into the
// mantissa of 1024.0, minus 1032) and then its FP6 E3M2 register image with
// one v_cvt_scalef32_pk32_bf6_f16 (exact on these integers), stored into the
// FP6 tile layout in LDS, one slice ahead, through a ring of three stages.
// From there the slice runs as in the FP6 kernel (same fragments, products
// and epilogue) on eight waves of 128 x 64 in two phase-alternating groups:
// one group reads its first 64-k step's fragments and expands its slots of
// the next slice while the other issues its products (reading its second
// step's fragments among them), so the expansion's vector work overlaps the
// partner's matrix-core work.  The last iterations reload and re-expand the
// final slice, so the loop body has no branches around its loads; a padded
// last slice (odd slice counts) is walked but not multiplied.
constexpr int kP4Tile = 1024;                          // bytes of one packed 32 x 64 tile

typedef _Float16 v32h __attribute__((ext_vector_type(32)));

// FP6 register image of one packed slot: element 8q + 2i (+1) is nibble i
// (i + 4) of word q.  lo / hi hold the even / odd nibbles of a word in their
// bytes; one byte permute against 0x64 bytes forms each fp16 pair
// (1024 + n, 1024 + n'), one packed subtract of (1032, 1032) the codes.
__device__ __forceinline__ v6u expand_slot(const uint4 &s) {
    const uint32_t w[4] = {s.x, s.y, s.z, s.w};
    const h2 off = __builtin_bit_cast(h2, 0x64086408u);   // (1032, 1032)
    const uint32_t c64 = 0x64646464u;
    v32h v;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const uint32_t lo = w[q] & 0x0F0F0F0Fu, hi = (w[q] >> 4) & 0x0F0F0F0Fu;
        // pair i: nibbles (i, i + 4) = (lo, hi alternating) bytes (i / 2, i / 2 + 2)
        const uint32_t pr[4] = {__builtin_amdgcn_perm(c64, lo, 0x04020400u), __builtin_amdgcn_perm(c64, hi, 0x04020400u),
                                __builtin_amdgcn_perm(c64, lo, 0x04030401u), __builtin_amdgcn_perm(c64, hi, 0x04030401u)};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const h2 d = __builtin_bit_cast(h2, pr[i]) - off;
            v[8 * q + 2 * i] = d[0];
            v[8 * q + 2 * i + 1] = d[1];
        }
    }
    return __builtin_amdgcn_cvt_scalef32_pk32_bf6_f16(v, 1.0f);
}

__device__ __forceinline__ void store_image(int8_t *tile, int l, const v6u &img) {
    *reinterpret_cast<uint4 *>(tile + 16 * l) = make_uint4(img[0], img[1], img[2], img[3]);
    *reinterpret_cast<uint2 *>(tile + 1024 + 8 * l) = make_uint2(img[4], img[5]);
}

template <int OUT>
__global__ __launch_bounds__(2 * LThreads, 1) void gemm_a4w4_packed_kernel(Params p, int tiles_m, int tiles_n) {
    constexpr int STAGE = 2 * kF6Op;
    constexpr int SLOTS = 2 * (LB / 32) * 64 / (2 * LThreads);   // slots per thread, operand and slice (2)
    constexpr int EPI_BYTES = 1024 + 8 * 128 * big_epitch(2);
    constexpr int NST = 3;                      // LDS stages of FP6 images
    constexpr int SMEM = NST * STAGE > EPI_BYTES ? NST * STAGE : EPI_BYTES;
    __shared__ __attribute__((aligned(1024))) int8_t smem[SMEM];

    const int lane = threadIdx.x % kWave, wave = wave_id();
    const int group = wave / 4;
    const int wm = wave % 2, wn = (wave / 2) % 4;
    int tm, tn;
    xcd_tile(blockIdx.x, tiles_m, tiles_n, kGroupM, tm, tn);
    const int64_t m0 = (int64_t)tm * LB, n0 = (int64_t)tn * LB;
    const int64_t ktiles = (p.k + 127) / 128 * 2;
    const int64_t nk = ktiles / 2;
    const int64_t nkp = (nk + 1) / 2 * 2;            // slices walked (a padded last one is not multiplied)
    const int64_t rows_a = (p.m + 31) / 32, rows_b = (p.n + 31) / 32;

    // Slot i of this thread in a slice is s = tid + 512 i: tile s / 64 =
    // tid / 64 + 8 i (32-row block tid / 128 + 4 i, 64-k half (tid / 64) % 2),
    // lane slot tid % 64.
    const int tid = (int)threadIdx.x, sl = tid % 64, half = (tid / 64) % 2;
    const uint8_t *srcA[SLOTS];
    const uint8_t *srcB[SLOTS];
#pragma unroll
    for (int i = 0; i < SLOTS; i++) {
        const int rt = tid / 128 + 4 * i;
        const int64_t ra = min(m0 / 32 + rt, rows_a - 1), rb = min(n0 / 32 + rt, rows_b - 1);
        srcA[i] = reinterpret_cast<const uint8_t *>(p.x) + (ra * ktiles + half) * kP4Tile + 16 * sl;
        srcB[i] = reinterpret_cast<const uint8_t *>(p.w) + (rb * ktiles + half) * kP4Tile + 16 * sl;
    }
    const int dbase = (tid / 64) * kF6Tile;   // LDS tile of slot 0; slot i is 8 i tiles further
    uint4 la[2][SLOTS], lb[2][SLOTS];         // slice s lives in register set s % 2
    auto load = [&](int64_t slice, auto S) __attribute__((always_inline)) {
        const int64_t off = (slice < nk ? slice : nk - 1) * 2 * kP4Tile;
#pragma unroll
        for (int i = 0; i < SLOTS; i++) {
            la[S][i] = load16_stream(srcA[i] + off);
            lb[S][i] = load16_stream(srcB[i] + off);
        }
    };
    auto expand = [&](int8_t *stage, auto S) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SLOTS; i++) {
            store_image(stage + dbase + 8 * i * kF6Tile, sl, expand_slot(la[S][i]));
            store_image(stage + kF6Op + dbase + 8 * i * kF6Tile, sl, expand_slot(lb[S][i]));
        }
    };

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = v16f{};

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    load(0, I0{});
    load(1, I1{});
    expand(smem, I0{});
    load(2, I0{});
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this thread's images of slice 0 are stored
    if (group == 1) barrier_only();
    // One slice: wait for the barrier (slice kt's images complete, the stage
    // expanded into below free), read its fragments, expand slice kt + 1 from
    // its register set into the other stage, load slice kt + 3 into the set
    // just freed; barrier; the products.
    auto step = [&](int64_t kt, auto S) __attribute__((always_inline)) {
        constexpr int SN = 1 - decltype(S)::value;   // register set of slice kt + 1
        barrier_only();
        const int8_t *cur = smem + (int)(kt % NST) * STAGE;
        int8_t *nxt = smem + (int)((kt + 1) % NST) * STAGE;
        v8i fa[4], fb[2];
        auto frags = [&](int st) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; i++) fa[i] = f6_frag(cur + ((wm * 4 + i) * 2 + st) * kF6Tile, lane);
#pragma unroll
            for (int j = 0; j < 2; j++) fb[j] = f6_frag(cur + kF6Op + ((wn * 2 + j) * 2 + st) * kF6Tile, lane);
        };
        frags(0);
        expand(nxt, std::integral_constant<int, SN>{});
        load(kt + 3, std::integral_constant<int, SN>{});
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): fragments in registers, images stored
        barrier_only();
        if (kt < nk) {
#pragma unroll
            for (int st = 0; st < 2; st++) {
                if (st == 1) frags(1);
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int j = 0; j < 2; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 3, 3, 0,
                                                                                    kF6Scale, 0, kF6Scale);
            }
        }
    };
    for (int64_t kt = 0; kt < nkp; kt += 2) {
        step(kt, I0{});
        step(kt + 1, I1{});
    }
    if (group == 0) barrier_only();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    big_epilogue<EPI_SCALARS, OUT>(p, acc, smem, m0, n0, wm, wn, wave, lane);
}

template <int OUT>
hipError_t launch_packed(const Params &p, hipStream_t st) {
    const int64_t tm = (p.m + LB - 1) / LB, tn = (p.n + LB - 1) / LB;
    if (tm * tn > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_a4w4_packed_kernel<OUT>), dim3((unsigned)(tm * tn)), dim3(2 * LThreads), 0, st, p,
                       (int)tm, (int)tn);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// General kernel
// ---------------------------------------------------------------------------
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int WM = 64, WN = 64;   // wave sub-tile
constexpr int TM = WM / 32, TN = WN / 32;   // 32 x 32 blocks per wave sub-tile

// Operand loads of the general kernel.  Rows past the matrix (m for x, n
// for w) are read clamped to its last row: their products only reach output
// rows or columns that are never stored.  Only k past the end must add
// nothing, so only x's chunks in the last, partial k-step are zeroed (MASK);
// w's bytes beside them may be any finite values.  With VEC (k % 16 == 0,
// and n % 4 == 0 for [k][n] weights) every load is one unconditional vector
// load from a clamped in-bounds address, with no branch around it, so the
// loads stay in flight across the products that follow.  Otherwise byte
// loads with zero fill.

// 16 bytes of row `row` of a [rows][k] int8 matrix at column kk.
template <bool VEC, bool MASK>
__device__ __forceinline__ uint4 load_row16(const int8_t *base, int64_t rows, int64_t k, int64_t row,
                                            int64_t kk) {
    if constexpr (VEC) {
        const int64_t r = row < rows ? row : rows - 1;
        if constexpr (!MASK) {
            return *reinterpret_cast<const uint4 *>(base + r * k + kk);
        } else {
            const uint4 v = *reinterpret_cast<const uint4 *>(base + r * k + (kk < k ? kk : k - 16));
            return kk < k ? v : make_uint4(0, 0, 0, 0);
        }
    } else {
        if (row >= rows) return make_uint4(0, 0, 0, 0);
        const int8_t *p = base + row * k + kk;
        uint32_t v[4] = {0, 0, 0, 0};
        // unrolled, so v stays in registers (a run-time index would put it in scratch)
#pragma unroll
        for (int j = 0; j < 16; j++)
            if (kk + j < k) v[j / 4] |= (uint32_t)(uint8_t)p[j] << (8 * (j % 4));
        return make_uint4(v[0], v[1], v[2], v[3]);
    }
}

// 4 k-rows x 4 n-columns of a [k][n] int8 matrix as 4 row words (byte j of
// word i: k-row kk + i, column nn + j).
template <bool VEC, bool MASK>
__device__ __forceinline__ void load_kn_4x4(const int8_t *w, int64_t n, int64_t k, int64_t kk,
                                            int64_t nn, uint32_t rowv[4]) {
    if constexpr (VEC) {
        const int64_t nc = nn < n ? nn : n - 4;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t kr = MASK && kk + i >= k ? k - 1 : kk + i;
            rowv[i] = *reinterpret_cast<const uint32_t *>(w + kr * n + nc);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t r = 0;
#pragma unroll
            for (int j = 0; j < 4; j++)
                if (kk + i < k && nn + j < n) r |= (uint32_t)(uint8_t)w[(kk + i) * n + nn + j] << (8 * j);
            rowv[i] = r;
        }
    }
}

// The 4 x 4 byte transpose of load_kn_4x4's row words: word j holds the 4
// consecutive k of column nn + j.  Done when the words are stored, so the
// loads stay in flight until then.
__device__ __forceinline__ uint32_t kn_column(const uint32_t rowv[4], int j) {
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) c |= ((rowv[i] >> (8 * j)) & 0xffu) << (8 * i);
    return c;
}

// KALL = 1: one 64-byte k-step staged at a time, the next step's loads in
// flight while the current one is multiplied.  KALL > 1 (k <= 64 KALL): every
// k-step's loads are issued at once and the whole k range is staged in LDS
// before any product, so a short-k product pays one memory latency instead
// of one per step.
template <bool NK, bool VEC, int EPI, int OUT, int KALL>
__global__ __launch_bounds__(kThreads) void gemm_i8_kernel(Params p) {
    constexpr int PITCH = KALL * BK + 16;   // LDS row stride in bytes
    __shared__ __attribute__((aligned(16))) int8_t As[BM * PITCH];
    __shared__ __attribute__((aligned(16))) int8_t Bs[BN * PITCH];

    to_batch(p);
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int wm = wave / 2, wn = wave % 2;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t nk = (p.k + BK - 1) / BK;

    // Register staging of k-step slots: A as 2 x 16 bytes, B likewise
    // ([n][k]) or two 4 x 4 byte blocks as row words ([k][n]).
    uint4 ra[KALL][2];
    uint4 rb[KALL][2];
    uint32_t rbt[KALL][2][4];

    // `mask` (std::true_type / false_type): the k-step runs past k
    // the lambdas are inlined so the slot arrays stay in registers
    auto gload = [&](int slot, int64_t k0, auto mask) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask)::value;
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int chunk = tid + c * kThreads;
            const int row = chunk / 4, c16 = chunk % 4;
            ra[slot][c] = load_row16<VEC, MASK>(p.x, p.m, p.k, m0 + row, k0 + 16 * c16);
            if (NK) {
                rb[slot][c] = load_row16<VEC, MASK>(p.w, p.n, p.k, n0 + row, k0 + 16 * c16);
            } else {
                const int n4 = chunk % 32, k4 = chunk / 32;
                load_kn_4x4<VEC, MASK>(p.w, p.n, p.k, k0 + 4 * k4, n0 + 4 * n4, rbt[slot][c]);
            }
        }
    };
    // the branch is uniform (scalar): either path keeps its loads in flight
    auto gload_step = [&](int slot, int64_t kt) __attribute__((always_inline)) {
        if ((kt + 1) * BK > p.k) gload(slot, kt * BK, std::true_type{});
        else gload(slot, kt * BK, std::false_type{});
    };
    // slot s goes to LDS columns [64 s, 64 s + 64) of each row
    auto sstore = [&](int slot, int col0) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int chunk = tid + c * kThreads;
            const int row = chunk / 4, c16 = chunk % 4;
            *reinterpret_cast<uint4 *>(As + row * PITCH + col0 + 16 * c16) = ra[slot][c];
            if (NK) {
                *reinterpret_cast<uint4 *>(Bs + row * PITCH + col0 + 16 * c16) = rb[slot][c];
            } else {
                const int n4 = chunk % 32, k4 = chunk / 32;
#pragma unroll
                for (int j = 0; j < 4; j++)
                    *reinterpret_cast<uint32_t *>(Bs + (4 * n4 + j) * PITCH + col0 + 4 * k4) =
                        kn_column(rbt[slot][c], j);
            }
        }
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) acc[i][j] = v16i{};

    // v_mfma_i32_32x32x32_i8 (the 16x16x64 form sustains about 60% of its
    // rate): lane l supplies row / column l % 32 and the 16 k bytes at
    // 16 (l / 32) of each 32-byte step.  Row pitch 16 mod 64 bytes: the 8
    // rows read together fall in distinct bank groups.
    const int fr = lane % 32;           // fragment row / column
    const int fk = 16 * (lane / 32);    // fragment k offset (bytes)
    auto compute = [&](int col0) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < BK / 32; s++) {
            v4i a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; i++)
                a[i] = *reinterpret_cast<const v4i *>(As + (wm * WM + i * 32 + fr) * PITCH + col0 + fk + 32 * s);
#pragma unroll
            for (int j = 0; j < TN; j++)
                b[j] = *reinterpret_cast<const v4i *>(Bs + (wn * WN + j * 32 + fr) * PITCH + col0 + fk + 32 * s);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
        }
    };

    if constexpr (KALL == 1) {
        gload_step(0, 0);
        sstore(0, 0);
        __syncthreads();
        for (int64_t kt = 0; kt < nk; kt++) {
            if (kt + 1 < nk) gload_step(0, kt + 1);
            compute(0);
            __syncthreads();
            if (kt + 1 < nk) {
                sstore(0, 0);
                __syncthreads();
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < KALL; s++)
            if (s < nk) gload_step(s, s);
#pragma unroll
        for (int s = 0; s < KALL; s++)
            if (s < nk) sstore(s, s * BK);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < KALL; s++)
            if (s < nk) compute(s * BK);
        __syncthreads();
    }

    // Epilogue: lane holds column fr of each 32x32 block and rows
    // 8 (r / 4) + 4 (lane / 32) + r % 4 of register r.
    Epilogue<EPI, OUT> ep;
    ep.init(p);
    ep.stage_rows(p, m0, BM, reinterpret_cast<float *>(As));
    __syncthreads();
    float cf[TN], cb[TN];
#pragma unroll
    for (int j = 0; j < TN; j++) {
        cf[j] = ep.col_factor(p, n0 + wn * WN + j * 32 + fr);
        cb[j] = ep.col_bias(p, n0 + wn * WN + j * 32 + fr);
    }
#pragma unroll
    for (int j = 0; j < TN; j++) {
        const int64_t col = n0 + wn * WN + j * 32 + fr;
        if (col >= p.n) continue;
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int local = wm * WM + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
                if (m0 + local < p.m) ep.store(p, m0 + local, col, acc[i][j][r], ep.row_factor(local), cf[j], cb[j]);
            }
    }
}

// ---------------------------------------------------------------------------
// Decode kernel: m <= 128 (see gemv_fits), [n][k] weights, k % 64 == 0
// ---------------------------------------------------------------------------
// The m token rows fill RB 16-row blocks of v_mfma_i32_16x16x64_i8 (rows past
// m repeat row 0 and are never stored; the kernel is bound by the weight
// bytes, so the idle rows cost nothing).  A workgroup owns NBLK blocks of 16
// output columns; its kGvWaves waves take turns over k blocks of 64 SPS
// bytes, each wave holding two register stages so the next block's weights
// are in flight while the current one is multiplied.  Lane l supplies row /
// column l % 16 and the 16 bytes at k 64 t + 16 (l / 16) of step t, read
// straight from the row-major operands (weights with non-temporal loads:
// each byte is used once).  The waves' int32 partials are summed in LDS in a
// fixed order: exact, hence deterministic.
constexpr int kGvWaves = 8;

template <int NBLK, int SPS, int RB>
struct GemvStage {
    v4i w[SPS][NBLK];
    v4i a[SPS][RB];
};

// All loads of k block kb from clamped, in-bounds addresses; a step past
// the end is masked at compute time.
//
// XT (SPS even, k % 128 == 0): x moves in whole cache lines.  Steps 2i and
// 2i + 1 cover 128 bytes of each row; their loads give lane l piece l % 8 of
// row 16b + 8u + l / 8 (u = 0, 1), and gemv_compute turns them into
// fragments through the wave's LDS block (x_pair_fragments).
template <int NBLK, int SPS, int RB, bool XT>
__device__ __forceinline__ void gemv_load(GemvStage<NBLK, SPS, RB> &st, const int8_t *const (&xrow)[RB],
                                          const int8_t *const (&wrow)[NBLK], int64_t kb, int64_t nsteps,
                                          const int8_t *__restrict__ x, int64_t m, int64_t k, int lane,
                                          const int8_t *const (&wcol)[2 * NBLK]) {
#pragma unroll
    for (int t = 0; t < SPS; t++) {
        const int64_t s = kb * SPS + t;
        const int64_t off = (s < nsteps ? s : nsteps - 1) * 64;
        if constexpr (XT) {
            // the pair's first step, clamped to the last pair (nsteps is even)
            const int64_t s0 = kb * SPS + (t & ~1);
            const int64_t poff = (s0 < nsteps ? s0 : nsteps - 2) * 64;
#pragma unroll
            for (int b = 0; b < RB; b++) {
                const int64_t r = 16 * b + 8 * (t & 1) + lane / 8;
                st.a[t][b] = *reinterpret_cast<const v4i *>(x + (r < m ? r : 0) * k + poff + 16 * (lane % 8));
            }
        } else {
#pragma unroll
            for (int b = 0; b < RB; b++) st.a[t][b] = *reinterpret_cast<const v4i *>(xrow[b] + off);
        }
#pragma unroll
        for (int j = 0; j < NBLK; j++) {
            if constexpr (XT) {
                // weights in whole lines too: column 16 j + 8 (t & 1) + lane / 8
                const int64_t s0 = kb * SPS + (t & ~1);
                const int64_t poff = (s0 < nsteps ? s0 : nsteps - 2) * 64;
                const uint4 v = load16_stream(wcol[2 * j + (t & 1)] + poff);
                st.w[t][j] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            } else {
                const uint4 v = load16_stream(wrow[j] + off);
                st.w[t][j] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
        }
    }
}

// Row pitch of a wave's LDS block for XT: 128 bytes of x plus 16, so the
// fragment reads of 16 rows fall in distinct banks.
constexpr int kRow128Pitch = 144;

// Whole-line pieces of steps 2i, 2i + 1 (as gemv_load leaves them) to the
// fragments of those steps: lane (r, q) gets bytes 64u + 16q of row 16b + r.
// Only the wave touches its block and its LDS operations complete in issue
// order; the fences keep the compiler from reordering them.
template <int RB>
__device__ __forceinline__ void x_pair_fragments(const v4i (&in0b)[RB], const v4i (&in1b)[RB], v4i (&frag)[2][RB],
                                                 uint8_t *xb, int lane) {
#pragma unroll
    for (int b = 0; b < RB; b++) {
        *reinterpret_cast<v4i *>(xb + (16 * b + lane / 8) * kRow128Pitch + 16 * (lane % 8)) = in0b[b];
        *reinterpret_cast<v4i *>(xb + (16 * b + 8 + lane / 8) * kRow128Pitch + 16 * (lane % 8)) = in1b[b];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
        for (int b = 0; b < RB; b++)
            frag[u][b] = *reinterpret_cast<const v4i *>(xb + (16 * b + lane % 16) * kRow128Pitch + 64 * u +
                                                         16 * (lane / 16));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int NBLK, int SPS, int RB, bool XT>
__device__ __forceinline__ void gemv_compute(const GemvStage<NBLK, SPS, RB> &st, v4i (&acc)[RB][NBLK], int64_t kb,
                                             int64_t nsteps, uint8_t *xb, int lane) {
    v4i xa[SPS][RB], wa[SPS][NBLK];
    if constexpr (XT) {
#pragma unroll
        for (int i = 0; i < SPS / 2; i++) {
            if constexpr (RB <= 4) {
                v4i f[2][RB];
                x_pair_fragments<RB>(st.a[2 * i], st.a[2 * i + 1], f, xb, lane);
#pragma unroll
                for (int b = 0; b < RB; b++) {
                    xa[2 * i][b] = f[0][b];
                    xa[2 * i + 1][b] = f[1][b];
                }
            } else {
                // more row blocks pass through the 16-row block one at a time
#pragma unroll
                for (int b = 0; b < RB; b++) {
                    v4i f[2][1];
                    x_pair_fragments<1>(reinterpret_cast<const v4i(&)[1]>(st.a[2 * i][b]),
                                        reinterpret_cast<const v4i(&)[1]>(st.a[2 * i + 1][b]), f, xb, lane);
                    xa[2 * i][b] = f[0][0];
                    xa[2 * i + 1][b] = f[1][0];
                }
            }
            v4i g[2][NBLK];
            x_pair_fragments<NBLK>(st.w[2 * i], st.w[2 * i + 1], g, xb, lane);
#pragma unroll
            for (int j = 0; j < NBLK; j++) {
                wa[2 * i][j] = g[0][j];
                wa[2 * i + 1][j] = g[1][j];
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < SPS; t++) {
#pragma unroll
            for (int b = 0; b < RB; b++) xa[t][b] = st.a[t][b];
#pragma unroll
            for (int j = 0; j < NBLK; j++) wa[t][j] = st.w[t][j];
        }
    }
#pragma unroll
    for (int t = 0; t < SPS; t++) {
        // a zero activation fragment removes a step past the end exactly
        const bool ok = kb * SPS + t < nsteps;
#pragma unroll
        for (int b = 0; b < RB; b++) {
            const v4i a = ok ? xa[t][b] : v4i{0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < NBLK; j++)
                acc[b][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, wa[t][j], acc[b][j], 0, 0, 0);
        }
    }
}

// Row factors of lane's output rows 16 b + 4 (lane / 16) + r of the decode
// kernels (rows past m repeat the last one; they are never stored).
template <int RB, int EPI, int OUT>
__device__ __forceinline__ void gemv_row_factors(const Params &p, const Epilogue<EPI, OUT> &ep, float (&rf)[RB][4],
                                                 int lane) {
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int64_t row = 16 * b + 4 * (lane / 16) + r < p.m ? 16 * b + 4 * (lane / 16) + r : p.m - 1;
            rf[b][r] = OUT == OUT_I32 ? 0.0f : (EPI == EPI_ROWCOL ? p.pts[row] : ep.sa);
        }
}

// The decode kernels' end: every wave's 16x16 int32 partials to LDS, then
// each output block summed over the WAVES waves in wave order (exact) and
// stored through the epilogue.  Lane l holds column l % 16 and rows
// 4 (l / 16) + r of a block; column blocks nb0 .. nb0 + NBLK - 1.
template <int WAVES, int RB, int NBLK, int EPI, int OUT>
__device__ __forceinline__ void gemv_reduce_store(const Params &p, const Epilogue<EPI, OUT> &ep,
                                                  const v4i (&acc)[RB][NBLK], v4i (*red)[RB * NBLK][kWave],
                                                  const float (&rf)[RB][4], int64_t nb0, int wave, int lane) {
    const int fr = lane % 16;
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int j = 0; j < NBLK; j++) red[wave][b * NBLK + j][lane] = acc[b][j];
    __syncthreads();
    for (int e = wave; e < RB * NBLK; e += WAVES) {
        const int b = e / NBLK, j = e % NBLK;
        const int64_t col = (nb0 + j) * 16 + fr;
        if (col >= p.n) continue;
        v4i sum = red[0][e][lane];
#pragma unroll
        for (int w = 1; w < WAVES; w++) sum += red[w][e][lane];
        const float cf = ep.col_factor(p, col), cb = ep.col_bias(p, col);
        float rfe[4];
#pragma unroll
        for (int r = 0; r < 4; r++) rfe[r] = rf[0][r];
#pragma unroll
        for (int bb = 1; bb < RB; bb++)
            if (bb == b)
#pragma unroll
                for (int r = 0; r < 4; r++) rfe[r] = rf[bb][r];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int64_t row = 16 * b + 4 * (lane / 16) + r;
            if (row < p.m) ep.store(p, row, col, sum[r], rfe[r], cf, cb);
        }
    }
}

template <int NBLK, int SPS, int RB, int EPI, int OUT, bool XT>
__global__ __launch_bounds__(kGvWaves * 64) void gemv_i8_kernel(Params p) {
    __shared__ v4i red[kGvWaves][RB * NBLK][kWave];
    constexpr int kXRows = RB <= 4 ? (RB > NBLK ? RB : NBLK) : NBLK;  // 16-row blocks in the wave's LDS block
    __shared__ __attribute__((aligned(16))) int8_t xlds[XT ? kGvWaves : 1][XT ? 16 * kXRows * kRow128Pitch : 16];
    to_batch(p);
    const int lane = threadIdx.x % kWave, wave = wave_id();
    uint8_t *xb = reinterpret_cast<uint8_t *>(xlds[XT ? wave : 0]);
    const int fr = lane % 16;
    const int64_t nb0 = (int64_t)blockIdx.x * NBLK;
    const int64_t nsteps = p.k / 64, kblocks = (nsteps + SPS - 1) / SPS;
    const int8_t *xrow[RB];
#pragma unroll
    for (int b = 0; b < RB; b++) {
        const int64_t row = 16 * b + fr;
        xrow[b] = p.x + (row < p.m ? row : 0) * p.k + 16 * (lane / 16);
    }
    // columns past n repeat the last one; they are never stored
    const int8_t *wrow[NBLK];
#pragma unroll
    for (int j = 0; j < NBLK; j++) {
        const int64_t col = (nb0 + j) * 16 + fr;
        wrow[j] = p.w + (col < p.n ? col : p.n - 1) * p.k + 16 * (lane / 16);
    }
    // whole-line weight loads (XT): column 16 j + 8 u + lane / 8, clamped
    const int8_t *wcol[2 * NBLK];
#pragma unroll
    for (int i = 0; i < 2 * NBLK; i++) {
        const int64_t col = (nb0 + i / 2) * 16 + 8 * (i % 2) + lane / 8;
        wcol[i] = p.w + (col < p.n ? col : p.n - 1) * p.k + 16 * (lane % 8);
    }
    // row factors of this lane's output rows, loaded now so their latency
    // hides behind the k loop
    Epilogue<EPI, OUT> ep;
    ep.init(p);
    float rf[RB][4];
    gemv_row_factors<RB>(p, ep, rf, lane);

    v4i acc[RB][NBLK];
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int j = 0; j < NBLK; j++) acc[b][j] = v4i{0, 0, 0, 0};
    GemvStage<NBLK, SPS, RB> s0, s1;
    int64_t kb = wave;
    if (kb < kblocks) gemv_load<NBLK, SPS, RB, XT>(s0, xrow, wrow, kb, nsteps, p.x, p.m, p.k, lane, wcol);
    while (kb < kblocks) {
        const int64_t kb1 = kb + kGvWaves;
        if (kb1 < kblocks) gemv_load<NBLK, SPS, RB, XT>(s1, xrow, wrow, kb1, nsteps, p.x, p.m, p.k, lane, wcol);
        gemv_compute<NBLK, SPS, RB, XT>(s0, acc, kb, nsteps, xb, lane);
        if (kb1 >= kblocks) break;
        const int64_t kb2 = kb1 + kGvWaves;
        if (kb2 < kblocks) gemv_load<NBLK, SPS, RB, XT>(s0, xrow, wrow, kb2, nsteps, p.x, p.m, p.k, lane, wcol);
        gemv_compute<NBLK, SPS, RB, XT>(s1, acc, kb1, nsteps, xb, lane);
        kb = kb2;
    }

    gemv_reduce_store<kGvWaves, RB, NBLK>(p, ep, acc, red, rf, nb0, wave, lane);
}

template <int NBLK, int SPS, int RB, int EPI, int OUT>
hipError_t launch_gemv_t(const Params &p, int64_t batch, hipStream_t st) {
    const int64_t nblocks = (p.n + 15) / 16;
    const dim3 grid((unsigned)((nblocks + NBLK - 1) / NBLK), 1, (unsigned)batch);
    // Whole-line x loads need pairs of 64-k steps in a stage and in k, and
    // an LDS block per wave (up to four row blocks).
    if constexpr (SPS % 2 == 0) {
        if (p.k % 128 == 0) {
            hipLaunchKernelGGL((gemv_i8_kernel<NBLK, SPS, RB, EPI, OUT, true>), grid, dim3(kGvWaves * 64), 0, st, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemv_i8_kernel<NBLK, SPS, RB, EPI, OUT, false>), grid, dim3(kGvWaves * 64), 0, st, p);
    return hipGetLastError();
}

// Launch shapes measured on MI355X with the weights streamed from HBM
// (HIP-graph replays rotating copies) against 1, 2, 4 and 7 column blocks per
// workgroup and 64-, 128- and 256-k stages, at n x k = 4096 x 4096,
// 11008 x 4096, 4096 x 11008 and 28672 x 8192.  One row block (m <= 16): one
// column block per workgroup, 256-k stages up to 384 column blocks, 128-k
// above (best or within 6% of best).  More row blocks re-read x for every
// column block a workgroup owns, so past 384 column blocks four of them
// share each x fragment (64-k stages keep the registers in bounds): the best
// measured shape at m = 32, 48 and 64.
template <int RB, int EPI, int OUT>
hipError_t launch_gemv_n(const Params &p, int64_t batch, hipStream_t st) {
    const int64_t nblocks = (p.n + 15) / 16;
    if constexpr (RB == 1) {
        if (nblocks <= 384) return launch_gemv_t<1, 4, RB, EPI, OUT>(p, batch, st);
        return launch_gemv_t<1, 2, RB, EPI, OUT>(p, batch, st);
    }
    if (nblocks <= 384) return launch_gemv_t<1, 2, RB, EPI, OUT>(p, batch, st);
    // two row blocks: 128-k stages (whole-line x) still fit in registers
    if (p.k % 128 == 0) {
        if constexpr (RB == 2) return launch_gemv_t<4, 2, RB, EPI, OUT>(p, batch, st);
        else return launch_gemv_t<2, 2, RB, EPI, OUT>(p, batch, st);
    }
    return launch_gemv_t<4, 1, RB, EPI, OUT>(p, batch, st);
}

template <int EPI, int OUT>
hipError_t launch_gemv_rb(const Params &p, int64_t batch, hipStream_t st) {
    switch ((p.m + 15) / 16) {
        case 1: return launch_gemv_n<1, EPI, OUT>(p, batch, st);
        case 2: return launch_gemv_n<2, EPI, OUT>(p, batch, st);
        case 3: return launch_gemv_n<3, EPI, OUT>(p, batch, st);
        case 4: return launch_gemv_n<4, EPI, OUT>(p, batch, st);
        // 64 < m <= 128, at most 384 column blocks (gemv_fits): six row blocks
        // take 128-k whole-line stages (k % 128 == 0), else 64-k stages
        case 5: case 6:
            if (p.k % 128 == 0) return launch_gemv_t<1, 2, 6, EPI, OUT>(p, batch, st);
            return launch_gemv_t<1, 1, 6, EPI, OUT>(p, batch, st);
        // (eight row blocks: 128-k stages no longer fit in registers)
        default: return launch_gemv_t<1, 1, 8, EPI, OUT>(p, batch, st);
    }
}

// ---------------------------------------------------------------------------
// Decode kernel for [k][n] weights: m <= 64, k % 64 == 0, n % 4 == 0
// ---------------------------------------------------------------------------
// The matrix cores take the weights as 16 consecutive k of one column per
// lane, which [k][n] rows do not hold.  A workgroup owns 16 NBLK columns;
// lane (q, c) of a 64-k step loads NBLK column dwords (4 NBLK columns from
// 4 NBLK c on) of rows 4 q .. 4 q + 3, transposes each 4 x 4 byte block in
// registers into 4-k column words, writes them to the wave's LDS block as
// [column][k] and reads whole 16-byte fragments back.  The x fragments come
// straight from the row-major activations, as in the [n][k] decode kernel.
// WAVES waves take turns over the 64-k steps, S steps at a time in flight in
// registers; their int32 partials are summed in LDS in wave order (exact).
// Workgroups are laid out so that each XCD (workgroup id mod 8) owns a
// contiguous run of column groups and its L2 serves neighbouring rows.
//
// LDS: column c's 64 k at c * 80 + (c / 16) * 64 bytes.  The 80-byte pitch
// puts the 16 fragment reads of a step in distinct banks, and the extra 64
// bytes per 16 columns spread the writes of the NBLK column blocks over
// distinct bank groups.
constexpr int kKnPitch = 80;
constexpr int kKnBlock = 16 * kKnPitch + 64;

__device__ __forceinline__ int kn_lds_col(int c) { return c * kKnPitch + (c / 16) * 64; }

template <int NBLK, int RB>
struct KnStage {
    static_assert(NBLK == 1 || NBLK == 4, "one column dword or one 16-byte piece per row and lane");
    v4i a[RB];
    uint32_t w[4][NBLK];   // rows 4 q + i, NBLK column dwords
};

template <int NBLK, int RB>
__device__ __forceinline__ void kn_load(KnStage<NBLK, RB> &st, const int8_t *const (&xrow)[RB], const int8_t *wblk,
                                        int64_t step, int64_t n) {
    const int64_t k0 = step * 64;
#pragma unroll
    for (int b = 0; b < RB; b++) st.a[b] = *reinterpret_cast<const v4i *>(xrow[b] + k0);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int8_t *src = wblk + (k0 + i) * n;
        if constexpr (NBLK == 4) {
            const uint4 v = load16_stream(src);
            st.w[i][0] = v.x; st.w[i][1] = v.y; st.w[i][2] = v.z; st.w[i][3] = v.w;
        } else {
            st.w[i][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(src));
        }
    }
}

template <int NBLK, int RB, int WAVES, int S, int EPI, int OUT>
__global__ __launch_bounds__(WAVES * 64) void gemv_kn_i8_kernel(Params p, int groups) {
    __shared__ v4i red[WAVES][RB * NBLK][kWave];
    __shared__ __attribute__((aligned(16))) uint8_t wt[WAVES][NBLK * kKnBlock];
    to_batch(p);
    const int lane = threadIdx.x % kWave, wave = wave_id();
    // XCD-contiguous column groups: workgroup b runs on XCD b % 8
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int per = groups / 8, rem = groups % 8;
    const int64_t nb0 = (int64_t)(xcd * per + min(xcd, rem) + slot) * NBLK;
    const int64_t nsteps = p.k / 64;

    const int8_t *xrow[RB];
#pragma unroll
    for (int b = 0; b < RB; b++) {
        const int64_t row = 16 * b + lane % 16;
        xrow[b] = p.x + (row < p.m ? row : 0) * p.k + 16 * (lane / 16);
    }
    // lane (q, c): rows 4 q + i of the step, columns 4 NBLK c .. + 4 NBLK - 1
    // of the group (past n: the last whole dwords, never stored)
    const int c = lane % 4, q = lane / 4;
    const int64_t wcol = min(nb0 * 16 + 4 * NBLK * c, p.n - 4 * NBLK);
    const int8_t *wblk = p.w + (int64_t)(4 * q) * p.n + wcol;
    uint8_t *wl = wt[wave];

    Epilogue<EPI, OUT> ep;
    ep.init(p);
    float rf[RB][4];
    gemv_row_factors<RB>(p, ep, rf, lane);

    v4i acc[RB][NBLK];
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int j = 0; j < NBLK; j++) acc[b][j] = v4i{0, 0, 0, 0};

    auto compute = [&](const KnStage<NBLK, RB> &st) __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < NBLK; d++) {
            const uint32_t rowv[4] = {st.w[0][d], st.w[1][d], st.w[2][d], st.w[3][d]};
#pragma unroll
            for (int j = 0; j < 4; j++)
                *reinterpret_cast<uint32_t *>(wl + kn_lds_col(4 * NBLK * c + 4 * d + j) + 4 * q) = kn_column(rowv, j);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        v4i wf[NBLK];
#pragma unroll
        for (int j = 0; j < NBLK; j++)
            wf[j] = *reinterpret_cast<const v4i *>(wl + kn_lds_col(16 * j + lane % 16) + 16 * (lane / 16));
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int b = 0; b < RB; b++)
#pragma unroll
            for (int j = 0; j < NBLK; j++)
                acc[b][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.a[b], wf[j], acc[b][j], 0, 0, 0);
    };

    // Rounds of S steps (wave + (i + S t) WAVES): all S steps' loads are
    // issued, then each step is multiplied as its loads land.  Loads are
    // unconditional (steps past the end re-read the last one and are not
    // multiplied), so each step's wait is a fixed count and no load is
    // carried across the loop's back edge.
    for (int64_t base = wave; base < nsteps; base += (int64_t)S * WAVES) {
        KnStage<NBLK, RB> st[S];
        static_for<0, S>([&](auto I) {
            const int64_t s0 = base + (int64_t)I * WAVES;
            kn_load<NBLK, RB>(st[I], xrow, wblk, s0 < nsteps ? s0 : nsteps - 1, p.n);
        });
        static_for<0, S>([&](auto I) {
            if (base + (int64_t)I * WAVES < nsteps) compute(st[I]);
        });
    }
    gemv_reduce_store<WAVES, RB, NBLK>(p, ep, acc, red, rf, nb0, wave, lane);
}

template <int NBLK, int RB, int WAVES, int S, int EPI, int OUT>
hipError_t launch_gemv_kn_t(const Params &p, int64_t batch, hipStream_t st) {
    const int64_t groups = ((p.n + 15) / 16 + NBLK - 1) / NBLK;
    if (groups > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemv_kn_i8_kernel<NBLK, RB, WAVES, S, EPI, OUT>), dim3((unsigned)groups, 1, (unsigned)batch),
                       dim3(WAVES * 64), 0, st, p, (int)groups);
    return hipGetLastError();
}

// Four column blocks (64-byte row segments, x read once per 64 columns)
// once that still makes 256 workgroups and n allows whole 16-byte loads;
// one column block with eight waves below that; at most four 64-k steps
// (a launch-bound product): four waves, one step each.
template <int RB, int EPI, int OUT>
hipError_t launch_gemv_kn_n(const Params &p, int64_t batch, hipStream_t st) {
    if (p.n % 16 == 0 && (p.n / 64) * batch >= 256) return launch_gemv_kn_t<4, RB, 4, 4, EPI, OUT>(p, batch, st);
    if (p.k / 64 <= 4) return launch_gemv_kn_t<1, RB, 4, 1, EPI, OUT>(p, batch, st);
    return launch_gemv_kn_t<1, RB, 8, 4, EPI, OUT>(p, batch, st);
}

template <int EPI, int OUT>
hipError_t launch_gemv_kn_rb(const Params &p, int64_t batch, hipStream_t st) {
    switch ((p.m + 15) / 16) {
        case 1: return launch_gemv_kn_n<1, EPI, OUT>(p, batch, st);
        case 2: return launch_gemv_kn_n<2, EPI, OUT>(p, batch, st);
        case 3: return launch_gemv_kn_n<3, EPI, OUT>(p, batch, st);
        default: return launch_gemv_kn_n<4, EPI, OUT>(p, batch, st);
    }
}

template <int EPI>
hipError_t launch_gemv_kn_out(int out_kind, const Params &p, int64_t batch, hipStream_t st) {
    switch (out_kind) {
        case OUT_F16: return launch_gemv_kn_rb<EPI, OUT_F16>(p, batch, st);
        case OUT_BF16: return launch_gemv_kn_rb<EPI, OUT_BF16>(p, batch, st);
        default: return launch_gemv_kn_rb<EPI, OUT_I32>(p, batch, st);
    }
}

// [k][n] products the decode kernel takes (whole 64-k steps, whole column
// dwords).
bool gemv_kn_fits(int64_t m, int64_t n, int64_t k) {
    return m <= 64 && k % 64 == 0 && n % 4 == 0;
}

// Products the decode kernel takes: m <= 64, or m <= 128 when the columns
// are few.  Past 64 rows every column block re-reads eight 16-row blocks of
// x; measured with the weights streamed from HBM, that beats the 128x128
// tiles only up to 384 column blocks (128x4096x4096 21.8 against 50.9 us;
// at n = 11008 the two tie, at 28672 the tiles win).
bool gemv_fits(int64_t m, int64_t n) {
    return m <= 64 || (m <= 128 && (n + 15) / 16 <= 384);
}

template <int EPI>
hipError_t launch_gemv_out(int out_kind, const Params &p, int64_t batch, hipStream_t st) {
    switch (out_kind) {
        case OUT_F16: return launch_gemv_rb<EPI, OUT_F16>(p, batch, st);
        case OUT_BF16: return launch_gemv_rb<EPI, OUT_BF16>(p, batch, st);
        default: return launch_gemv_rb<EPI, OUT_I32>(p, batch, st);
    }
}

constexpr int kShortSteps = 4;   // k <= 256: the whole k range staged at once

template <bool NK, bool VEC, int EPI, int OUT>
hipError_t launch_t(const Params &p, int64_t batch, hipStream_t st) {
    dim3 grid((unsigned)((p.n + BN - 1) / BN), (unsigned)((p.m + BM - 1) / BM), (unsigned)batch);
    // (the byte-load form stages one k-step at a time: its staging registers
    // for the whole k range would not fit)
    if constexpr (VEC) {
        if (p.k <= (int64_t)kShortSteps * BK) {
            hipLaunchKernelGGL((gemm_i8_kernel<NK, VEC, EPI, OUT, kShortSteps>), grid, dim3(kThreads), 0, st, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_i8_kernel<NK, VEC, EPI, OUT, 1>), grid, dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

constexpr int kBigBK = 64;     // k bytes per slice
constexpr int kBigBuf = 3;     // slices in the LDS ring (two in flight ahead)

template <int EPI, int OUT>
hipError_t launch_big(const Params &p, int64_t batch, hipStream_t st) {
    const int tiles_m = (int)((p.m + LB - 1) / LB), tiles_n = (int)((p.n + LB - 1) / LB);
    hipLaunchKernelGGL((gemm_i8_big_kernel<kBigBK, kBigBuf, EPI, OUT>),
                       dim3((unsigned)(tiles_m * tiles_n), 1, (unsigned)batch), dim3(2 * LThreads), 0, st, p,
                       tiles_m, tiles_n);
    return hipGetLastError();
}

template <bool NK, bool VEC, int EPI>
hipError_t launch_out(int out_kind, const Params &p, int64_t batch, hipStream_t st) {
    switch (out_kind) {
        case OUT_F16: return launch_t<NK, VEC, EPI, OUT_F16>(p, batch, st);
        case OUT_BF16: return launch_t<NK, VEC, EPI, OUT_BF16>(p, batch, st);
        default: return launch_t<NK, VEC, EPI, OUT_I32>(p, batch, st);
    }
}

template <int EPI>
hipError_t launch_big_out(int out_kind, const Params &p, int64_t batch, hipStream_t st) {
    switch (out_kind) {
        case OUT_F16: return launch_big<EPI, OUT_F16>(p, batch, st);
        case OUT_BF16: return launch_big<EPI, OUT_BF16>(p, batch, st);
        default: return launch_big<EPI, OUT_I32>(p, batch, st);
    }
}

template <bool NK, bool VEC>
hipError_t launch_epi(int epi, int out_kind, const Params &p, int64_t batch, hipStream_t st) {
    return epi == EPI_ROWCOL ? launch_out<NK, VEC, EPI_ROWCOL>(out_kind, p, batch, st)
                             : launch_out<NK, VEC, EPI_SCALARS>(out_kind, p, batch, st);
}

}  // namespace

hipError_t launch_gemm_a4w4_packed(const uint8_t *xa, const uint8_t *wb, const float *sa, const float *sw, float eps,
                                   int64_t m, int64_t n, int64_t k, int out_kind, void *out, hipStream_t st) {
    Params p{reinterpret_cast<const int8_t *>(xa), reinterpret_cast<const int8_t *>(wb), nullptr, nullptr, sa, sw,
             eps, m, n, k, out, nullptr, 0, 0, 0, 0, 0};
    switch (out_kind) {
        case OUT_F16: return launch_packed<OUT_F16>(p, st);
        case OUT_BF16: return launch_packed<OUT_BF16>(p, st);
        default: return launch_packed<OUT_I32>(p, st);
    }
}

hipError_t launch_gemm_a4w4_tiles(const uint8_t *xa, const uint8_t *wb, const float *sa, const float *sw, float eps,
                                  int64_t m, int64_t n, int64_t k, int out_kind, void *out, hipStream_t st) {
    Params p{reinterpret_cast<const int8_t *>(xa), reinterpret_cast<const int8_t *>(wb), nullptr, nullptr, sa, sw,
             eps, m, n, k, out, nullptr, 0, 0, 0, 0, 0};
    switch (out_kind) {
        case OUT_F16: return launch_f6<OUT_F16>(p, st);
        case OUT_BF16: return launch_f6<OUT_BF16>(p, st);
        default: return launch_f6<OUT_I32>(p, st);
    }
}

// The large tiles need at least 128 of them per launch: measured with
// [n][k] weights at k = 4096, us, 256 x 256 against 128 x 128 tiles:
// 512x4096 56.5 / 40.6, 1024x4096 57.9 / 44.5, 2048x4096 62.2-63.2 /
// 61.2 (128 tiles), 1024x11008 71.2-72.0 / 86.4 (172 tiles), 4096x4096
// 84.4 / 120 (256 tiles).
bool gemm_i8_uses_big_tiles(bool w_nk, int64_t m, int64_t n, int64_t k, int64_t batch) {
    const int64_t tiles = ((m + LB - 1) / LB) * ((n + LB - 1) / LB);
    return w_nk && (k % kBigBK) == 0 && m >= 2 * LB && n >= 2 * LB && tiles <= 0x7fffffff && tiles * batch >= 128;
}

hipError_t launch_gemm_i8(const GemmI8Args &a, hipStream_t st) {
    const int64_t batch = a.batch < 1 ? 1 : a.batch;
    if (batch > 65535) return hipErrorInvalidValue;
    const int64_t es = a.out_kind == OUT_I32 ? 4 : 2;
    Params p{a.x, a.w, a.pts, a.deq, a.sa, a.sw, a.eps, a.m, a.n, a.k, a.out, a.bias,
             a.m * a.k, a.n * a.k, a.m, a.deq_stride, a.m * a.n * es};
    if (a.w_nk && gemv_fits(a.m, a.n) && a.k % 64 == 0) {
        if ((a.n + 15) / 16 > 0x7fffffff) return hipErrorInvalidValue;
        return a.epi == EPI_ROWCOL ? launch_gemv_out<EPI_ROWCOL>(a.out_kind, p, batch, st)
                                   : launch_gemv_out<EPI_SCALARS>(a.out_kind, p, batch, st);
    }
    if (!a.w_nk && gemv_kn_fits(a.m, a.n, a.k)) {
        if ((a.n + 15) / 16 > 0x7fffffff) return hipErrorInvalidValue;
        return a.epi == EPI_ROWCOL ? launch_gemv_kn_out<EPI_ROWCOL>(a.out_kind, p, batch, st)
                                   : launch_gemv_kn_out<EPI_SCALARS>(a.out_kind, p, batch, st);
    }
    if (gemm_i8_uses_big_tiles(a.w_nk, a.m, a.n, a.k, batch))
        return a.epi == EPI_ROWCOL ? launch_big_out<EPI_ROWCOL>(a.out_kind, p, batch, st)
                                   : launch_big_out<EPI_SCALARS>(a.out_kind, p, batch, st);
    if (a.m > (int64_t)BM * 65535) return hipErrorInvalidValue;
    // whole 16-byte rows of x and w ([n][k]), whole 4-column words of w ([k][n])
    const bool vec = (a.k % 16) == 0 && (a.w_nk || (a.n % 4) == 0);
    if (a.w_nk)
        return vec ? launch_epi<true, true>(a.epi, a.out_kind, p, batch, st)
                   : launch_epi<true, false>(a.epi, a.out_kind, p, batch, st);
    return vec ? launch_epi<false, true>(a.epi, a.out_kind, p, batch, st)
               : launch_epi<false, false>(a.epi, a.out_kind, p, batch, st);
}

}  // namespace ql
