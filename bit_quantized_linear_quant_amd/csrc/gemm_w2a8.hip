// BitLinear product on 2-bit packed ternary weights, gfx950
// ("Class BitLinear" forward steps 4-5: integer codes times ternary codes,
// then the per-token activation scale and the scalar weight scale).
//
// The packed layout (16 columns x 256 k per 1 KB block, 16 bytes per lane)
// is fragment-ordered: word t of lane l is exactly the 16-k B operand of
// lane l in v_mfma_i32_16x16x64_i8 step t, so weights go straight from HBM
// into registers and are unpacked there -- (word >> 2a) & 0x03030303 is four
// consecutive k as bytes code+1 in {0,1,2} -- with no dequantized weight in
// memory.  The A operand of lane l in step t is the 16 bytes of its token
// row at k = 256kb + 64(l/16) + 16t, the same k assignment, so the matrix
// core sums matching terms.  The accumulator holds sum x*(code+1); the
// epilogue subtracts the token's code sum: acc = sum x*code exactly.
//
// m > 64: 128 x 256 tiles on v_mfma_i32_32x32x32_i8, eight waves in two
//         phase-alternating groups; activation codes and packed weights
//         streamed into LDS through a ring of 128-k slices; each lane takes
//         its weight words from LDS in the order the 32x32x32 operand needs.
//         Except, for k >= 2048 and at most 1024 column blocks, m <= 96 (the
//         decode kernel with six row blocks) and m <= 128 (two decode
//         launches of 64 and m - 64 rows).
// m <= 64: decode GEMV.  The m rows fill one to four 16-row MFMA blocks
//         (rows past m repeat row 0 and are never stored); each workgroup
//         owns NBLK column blocks and its waves split k, each wave keeping two
//         register stages so the next k block's weights are in flight while
//         the current one is multiplied; int32 partials are summed in LDS in
//         a fixed order (exact, hence deterministic).  Weights are read with
//         non-temporal loads: each byte is used exactly once.
#include "ql_device.hpp"
#include "ql_launch.hpp"

namespace ql {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v4i unpack_tern(uint32_t w) {
    return v4i{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u), (int)((w >> 4) & 0x03030303u),
               (int)((w >> 6) & 0x03030303u)};
}

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int t) {
    return t == 0 ? v.x : (t == 1 ? v.y : (t == 2 ? v.z : v.w));
}

__device__ __forceinline__ float dequant_value(int32_t v, float pts, float g, const float *bias, float cb) {
    const float y = __fmul_rn(__fmul_rn((float)v, pts), g);
    return bias ? __fadd_rn(y, cb) : y;   // the bias (if any) is added after the dequant
}

template <int OUT>
__device__ __forceinline__ void epilogue_store(void *out, int64_t idx, int32_t acc, int32_t rs,
                                               float pts, float g, const float *bias, float cb) {
    const int32_t v = acc - rs;
    if (OUT == OUT_I32) static_cast<int32_t *>(out)[idx] = v;
    else store_out<OUT>(out, idx, dequant_value(v, pts, g, bias, cb));
}

// Code sums and per-token scales of a tile's rows, staged in LDS after the
// main loop (every thread of the workgroup calls this; a barrier must follow)
// so no output element waits on a global load of its own.
template <int OUT>
__device__ __forceinline__ void stage_rows(const float *__restrict__ pts, const int32_t *__restrict__ rowsum,
                                           int64_t m, int64_t m0, int rows, int32_t *rs_lds, float *pts_lds) {
    for (int r = threadIdx.x; r < rows; r += blockDim.x) {
        const int64_t row = m0 + r < m ? m0 + r : m - 1;
        rs_lds[r] = rowsum[row];
        if (OUT != OUT_I32) pts_lds[r] = pts[row];
    }
}

// ---------------------------------------------------------------------------
// m > 64: large-tile GEMM
// ---------------------------------------------------------------------------
// A 512-thread workgroup owns a 128 x 256 output tile: eight waves, two per
// SIMD (waves w and w + 4 share SIMD w % 4), each owning a 64 x 64 part
// (2 x 4 of them) as 2 x 2 blocks of v_mfma_i32_32x32x32_i8 (the 16x16x64
// form sustains about 60% of the 32x32x32 rate on gfx950).  The tile is
// wide in n because the activation codes are the heavy operand: every
// tile column re-reads them, while the 2-bit weights cost a quarter of a
// byte per element.  The k loop runs over 128-k slices through a ring of
// six LDS stages of 24 KB.  Slice sl = 2 kb + hh holds half hh of k block
// kb:
//   * the activation codes of k 128 sl .. +127 (128 rows x 128 bytes, 16 KB)
//     go HBM -> LDS with global_load_lds_dwordx4; 16-byte chunk c of row r
//     sits at chunk position c ^ ((r >> 1) & 7), so each 16 lanes of a
//     fragment read (16 rows, two per bank group parity) fall in distinct
//     bank groups;
//   * packed lanes 32 hh .. 32 hh + 31 of each of the tile's sixteen
//     fragment blocks (the k groups 2 hh and 2 hh + 1, 512 contiguous bytes
//     each), one 1 KB direct load per wave.
// Step t (0..3) of a slice gives lane half h = lane / 32 the k group
// g = 2 hh + h and the weight word t: for the A operand, the 16 codes of
// chunk 4 h + t of its slice row (k = 256 kb + 64 g + 16 t); for B, word t of
// packed lane (column % 16) + 16 g, unpacked in registers.  Both operands
// take the same 16 k, so the matrix core sums matching terms.
//
// The groups of waves 0-3 and 4-7 run opposite phases of every slice: one
// reads its fragments of the slice from LDS and issues its share of the
// direct loads five slices ahead while the other unpacks its weight words
// and issues its 16 matrix-core products, so the matrix cores of a SIMD
// see a ready wave at every phase.  Two workgroup barriers per slice keep
// the phases apart; the second group passes one extra barrier at the start
// and the first group one at the end.  Before every barrier a wave waits
// until at most four slices of its own loads are in flight: a slice has
// landed (every wave's loads) at the barrier before its first read, and
// the ring is never overwritten while a partner still reads it.
constexpr int XBM = 128, XBN = 256, XBK = 128;
constexpr int kXGroupM = 4;
constexpr int kXBuf = 6;                               // ring stages
constexpr int kXASlice = XBM * XBK;                    // bytes of activation codes per slice
constexpr int kXBSlice = XBN / 16 * 512;               // bytes of packed weights per slice
constexpr int kXStage = kXASlice + kXBSlice;
constexpr int kPThreads = 512;
constexpr int kPLoads = kXASlice / 1024 / (kPThreads / kWave);   // 1 KB A loads per wave per slice (2)
static_assert(kXBSlice == 1024 * 8, "one 1 KB weight load for each wave per slice");
static_assert(kPLoads == 2, "the A load layout below assumes two 1 KB loads per wave and slice");

// Bytes of LDS the epilogue of a 128 x 256 tile uses: the rows' code sums
// and scales, then a padded 64 x 64 output tile per wave.
template <int OUT>
constexpr int xepi_bytes() {
    return 2 * XBM * 4 + 8 * 64 * (64 * (OUT == OUT_I32 || OUT == OUT_F32 ? 4 : 2) + 16);
}

template <int OUT>
__global__ __launch_bounds__(kPThreads, 1) void w2a8_big_kernel(const int8_t *__restrict__ xq,
                                                               const float *__restrict__ pts,
                                                               const int32_t *__restrict__ rowsum,
                                                               const uint32_t *__restrict__ packed,
                                                               const double *__restrict__ gamma,
                                                               const float *__restrict__ bias,
                                                               int64_t m, int64_t n, int64_t k,
                                                               void *__restrict__ out, int tiles_m,
                                                               int tiles_n) {
    constexpr int SMEM = kXBuf * kXStage > xepi_bytes<OUT>() ? kXBuf * kXStage : xepi_bytes<OUT>();
    __shared__ __attribute__((aligned(1024))) int8_t smem[SMEM];
    const int lane = threadIdx.x % kWave, wave = wave_id();
    const int group = wave / 4;
    const int wm = wave % 2, wn = wave / 2;   // 2 x 4 quarters of 64 x 64
    int tm, tn;
    xcd_tile(blockIdx.x, tiles_m, tiles_n, kXGroupM, tm, tn);
    const int64_t m0 = (int64_t)tm * XBM, n0 = (int64_t)tn * XBN;
    const int64_t nsl = k / XBK, nblocks = n / 16;

    // A load ii of this wave fills LDS bytes [1024 (2 wave + ii), +1024) of
    // the slice: row 8 (2 wave + ii) + lane / 8, chunk position lane % 8.
    const int8_t *srca[kPLoads];
#pragma unroll
    for (int ii = 0; ii < kPLoads; ii++) {
        const int row = 8 * (kPLoads * wave + ii) + lane / 8;
        const int c = (lane % 8) ^ ((row >> 1) & 7);
        const int64_t r = m0 + row < m ? m0 + row : m - 1;
        srca[ii] = xq + r * k + 16 * c;
    }
    // Every wave loads weights: 32 lanes each in fragment blocks 2 wave and
    // 2 wave + 1 of the tile (half hh of k block kb at byte 512 sl).
    const int8_t *srcb;
    {
        const int blk = 2 * wave + lane / 32;
        const int64_t nb = n0 / 16 + blk < nblocks ? n0 / 16 + blk : nblocks - 1;
        srcb = reinterpret_cast<const int8_t *>(packed) + nb * (k / 256) * 1024 + 16 * (lane % 32);
    }
    const int h = lane / 32, fr = lane % 32;
    const int aoff = (64 * wm + fr) * XBK + 16 * ((4 * h) ^ ((fr >> 1) & 7));
    const int boff = kXASlice + 512 * (4 * wn + fr / 16) + 16 * (fr % 16 + 16 * h);

    auto issue = [&](int64_t sl, int stage) __attribute__((always_inline)) {
        const int64_t s = sl < nsl ? sl : nsl - 1;
        int8_t *dst = smem + stage * kXStage;
#pragma unroll
        for (int ii = 0; ii < kPLoads; ii++) lds_load16(srca[ii] + s * XBK, dst + 1024 * (kPLoads * wave + ii));
        lds_load16(srcb + s * 512, dst + kXASlice + 1024 * wave);
    };
    // at most four slices of this wave's loads in flight
    auto wait_ring = [&]() __attribute__((always_inline)) { wait_vmcnt<(kXBuf - 2) * (kPLoads + 1)>(); };

    v16i acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = v16i{};

#pragma unroll
    for (int i = 0; i < kXBuf - 1; i++) issue(i, i);
    if (group == 1) {
        wait_ring();
        barrier_only();
    }
    for (int64_t sl = 0; sl < nsl; sl++) {
        // fragment phase: this slice to registers, slice sl + 5 requested
        wait_ring();
        barrier_only();
        const int8_t *cur = smem + (int)(sl % kXBuf) * kXStage;
        v4i fa[4][2];
        uint4 bw[2];
#pragma unroll
        for (int j = 0; j < 2; j++) bw[j] = *reinterpret_cast<const uint4 *>(cur + boff + 1024 * j);
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
            for (int i = 0; i < 2; i++) fa[t][i] = *reinterpret_cast<const v4i *>(cur + (aoff ^ (16 * t)) + i * 32 * XBK);
        issue(sl + kXBuf - 1, (int)((sl + kXBuf - 1) % kXBuf));
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the fragments are in registers
        wait_ring();
        barrier_only();
        // product phase
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const v4i b = unpack_tern(word_of(bw[j], t));
#pragma unroll
                for (int i = 0; i < 2; i++)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[t][i], b, acc[i][j], 0, 0, 0);
            }
    }
    if (group == 0) barrier_only();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Epilogue through LDS: each wave converts its 64 x 64 sub-tile into an
    // LDS tile (rows padded by 16 bytes, so the four row groups of one write
    // fall in distinct banks), then writes whole 128- or 256-byte row
    // segments to global memory, 16 bytes per lane.
    int32_t *rs_lds = reinterpret_cast<int32_t *>(smem);
    float *pts_lds = reinterpret_cast<float *>(smem) + XBM;
    stage_rows<OUT>(pts, rowsum, m, m0, XBM, rs_lds, pts_lds);
    __syncthreads();
    constexpr int ES = OUT == OUT_I32 || OUT == OUT_F32 ? 4 : 2;   // output element bytes
    constexpr int ROWB = 64 * ES;                                  // bytes of a sub-tile row
    constexpr int PITCH = ROWB + 16;
    int8_t *tile = smem + 2 * XBM * 4 + wave * 64 * PITCH;
    const float g = OUT == OUT_I32 ? 0.0f : (float)gamma[0];  // gamma may be NULL for int32 output
    float cbj[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int64_t col = n0 + 64 * wn + 32 * j + fr;
        cbj[j] = (OUT != OUT_I32 && bias) ? bias[col < n ? col : n - 1] : 0.0f;
    }
    // Lane l holds column l % 32 of each 32 x 32 block and rows
    // 8 (r / 4) + 4 (l / 32) + r % 4 of register r.
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int lr = 32 * i + 8 * (r / 4) + 4 * h + r % 4;      // row within the sub-tile
            const int local = 64 * wm + lr;
            const float rf = OUT == OUT_I32 ? 0.0f : pts_lds[local];
            const int32_t rsv = rs_lds[local];
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int c = 32 * j + fr;
                const int32_t v = acc[i][j][r] - rsv;
                int8_t *dst = tile + lr * PITCH + c * ES;
                if constexpr (OUT == OUT_I32) *reinterpret_cast<int32_t *>(dst) = v;
                else if constexpr (OUT == OUT_F32) *reinterpret_cast<float *>(dst) = dequant_value(v, rf, g, bias, cbj[j]);
                else if constexpr (OUT == OUT_F16) *reinterpret_cast<uint16_t *>(dst) = f32_to_f16_rne(dequant_value(v, rf, g, bias, cbj[j]));
                else *reinterpret_cast<uint16_t *>(dst) = f32_to_bf16_rne(dequant_value(v, rf, g, bias, cbj[j]));
            }
        }
    // the wave reads back only its own sub-tile: a wave-local LDS ordering
    // (all lanes' writes complete) is enough
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    constexpr int SEG = ROWB / 16;                 // 16-byte pieces per sub-tile row
    constexpr int ROWS_PER = 64 / SEG;             // sub-tile rows per wave store
    const int64_t col0 = n0 + 64 * wn;
#pragma unroll
    for (int q = 0; q < 64 / ROWS_PER; q++) {
        const int lr = q * ROWS_PER + lane / SEG, piece = lane % SEG;
        const uint4 v = *reinterpret_cast<const uint4 *>(tile + lr * PITCH + 16 * piece);
        const int64_t row = m0 + 64 * wm + lr;
        const int64_t col = col0 + piece * (16 / ES);
        if (row < m && col < n) *reinterpret_cast<uint4 *>(static_cast<int8_t *>(out) + (row * n + col) * ES) = v;
    }
}

// ---------------------------------------------------------------------------
// m <= 16: split-K decode GEMV
// ---------------------------------------------------------------------------
// U k blocks of operands for the NBLK column blocks and RB row blocks of one
// wave.
template <int NBLK, int U, int RB>
struct GemvStage {
    uint4 w[U][NBLK];
    v4i a[U][RB][4];
};

// Issue every load of the k blocks kb0, kb0 + WAVES, ... (U of them) from
// clamped, in-bounds addresses; nothing is conditional, so no load waits for
// another.  A k block past the end is masked at compute time.
template <int NBLK, int WAVES, int U, int RB, bool XT>
__device__ __forceinline__ void gemv_load(GemvStage<NBLK, U, RB> &st, const int8_t *const (&xrow)[RB],
                                          const uint32_t *__restrict__ packed, int64_t kb0, int64_t nb0,
                                          int64_t nblocks, int64_t kblocks, int lane, const bool (&row_live)[RB],
                                          const int8_t *__restrict__ xq, int64_t m, int64_t k) {
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int64_t kb = kb0 + (int64_t)u * WAVES;
        const int64_t kbc = kb < kblocks ? kb : kblocks - 1;
#pragma unroll
        for (int j = 0; j < NBLK; j++) {
            const int64_t nbc = nb0 + j < nblocks ? nb0 + j : nblocks - 1;
            st.w[u][j] = load16_stream(packed + (nbc * kblocks + kbc) * 256 + 4 * lane);
        }
#pragma unroll
        for (int b = 0; b < RB; b++)
#pragma unroll
            for (int t = 0; t < 4; t++) {
                if constexpr (XT) {
                    // whole-line loads for rows256_to_fragments; rows past m
                    // read row 0 (their outputs are never stored)
                    const int64_t r = 16 * b + 4 * t + lane / 16;
                    st.a[u][b][t] =
                        *reinterpret_cast<const v4i *>(xq + (r < m ? r : 0) * k + kbc * 256 + 16 * (lane % 16));
                } else {
                    // lanes of rows past m load nothing (their rows are never stored)
                    st.a[u][b][t] = row_live[b] ? *reinterpret_cast<const v4i *>(xrow[b] + kbc * 256 + 16 * t)
                                                : v4i{0, 0, 0, 0};
                }
            }
    }
}

template <int NBLK, int WAVES, int U, int RB, bool XT>
__device__ __forceinline__ void gemv_compute(const GemvStage<NBLK, U, RB> &st, v4i (&acc)[RB][NBLK], int64_t kb0,
                                             int64_t kblocks, uint8_t *xb, int lane) {
#pragma unroll
    for (int u = 0; u < U; u++) {
        // a zero activation fragment removes a k block past the end exactly
        const bool ok = kb0 + (int64_t)u * WAVES < kblocks;
        v4i xa[RB][4];
        if constexpr (XT) {
            // one row block at a time through the wave's 16-row LDS block
#pragma unroll
            for (int b = 0; b < RB; b++)
                rows256_to_fragments<1>(reinterpret_cast<const v4i(&)[1][4]>(st.a[u][b]),
                                        reinterpret_cast<v4i(&)[1][4]>(xa[b]), xb, lane);
        } else {
#pragma unroll
            for (int b = 0; b < RB; b++)
#pragma unroll
                for (int t = 0; t < 4; t++) xa[b][t] = st.a[u][b][t];
        }
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
            for (int j = 0; j < NBLK; j++) {
                const v4i w = unpack_tern(word_of(st.w[u][j], t));
#pragma unroll
                for (int b = 0; b < RB; b++) {
                    const v4i a = ok ? xa[b][t] : v4i{0, 0, 0, 0};
                    acc[b][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, w, acc[b][j], 0, 0, 0);
                }
            }
    }
}

template <int NBLK, int WAVES, int U, int RB, int OUT, bool XT>
__global__ __launch_bounds__(WAVES * 64) void w2a8_gemv_kernel(const int8_t *__restrict__ xq,
                                                               const float *__restrict__ pts,
                                                               const int32_t *__restrict__ rowsum,
                                                               const uint32_t *__restrict__ packed,
                                                               const double *__restrict__ gamma,
                                                               const float *__restrict__ bias,
                                                               int64_t m, int64_t n, int64_t k,
                                                               void *__restrict__ out) {
    __shared__ v4i red[WAVES][RB * NBLK][kWave];
    // XT: x reaches the lanes through each wave's LDS block (whole-line loads)
    __shared__ __attribute__((aligned(16))) uint8_t xlds[XT ? WAVES : 1][XT ? 16 * kRow256Pitch : 16];
    const int lane = threadIdx.x % kWave, wave = wave_id();
    uint8_t *xb = xlds[XT ? wave : 0];
    const int64_t nb0 = (int64_t)blockIdx.x * NBLK;
    const int64_t nblocks = n / 16, kblocks = k / 256;
    const int fr = lane % 16;
    // Rows past m read row 0: an MFMA row only feeds its own output row,
    // which is never stored.  Column blocks past n likewise repeat the last.
    const int8_t *xrow[RB];
    bool row_live[RB];
#pragma unroll
    for (int b = 0; b < RB; b++) {
        row_live[b] = 16 * b + fr < m;
        xrow[b] = xq + (int64_t)(row_live[b] ? 16 * b + fr : 0) * k + 64 * (lane / 16);
    }
    // With one row block, this lane's output rows 4(lane/16) + r have their
    // code sums and scales loaded now, so their latency hides behind the k
    // loop; more row blocks load them in the epilogue, keeping the registers
    // for the operand stages.
    int32_t rsr[4];
    float ptr[4];
    if constexpr (RB == 1) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int64_t row = 4 * (lane / 16) + r < m ? 4 * (lane / 16) + r : m - 1;
            rsr[r] = rowsum[row];
            ptr[r] = OUT == OUT_I32 ? 0.0f : pts[row];
        }
    }

    v4i acc[RB][NBLK];
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int j = 0; j < NBLK; j++) acc[b][j] = v4i{0, 0, 0, 0};

    // Two register stages of U k blocks each: the loads of the next stage are
    // in flight while the matrix cores consume the current one.  U >= 4: one
    // stage holds every k block of the wave (the host launches it only when
    // kblocks <= WAVES * U), all loads issued at the start.
    constexpr int64_t step = (int64_t)WAVES * U;
    if constexpr (U >= 4) {
        GemvStage<NBLK, U, RB> s0;
        gemv_load<NBLK, WAVES, U, RB, XT>(s0, xrow, packed, wave, nb0, nblocks, kblocks, lane, row_live, xq, m, k);
        gemv_compute<NBLK, WAVES, U, RB, XT>(s0, acc, wave, kblocks, xb, lane);
    } else {
    GemvStage<NBLK, U, RB> s0, s1;
    int64_t kb = wave;
    gemv_load<NBLK, WAVES, U, RB, XT>(s0, xrow, packed, kb, nb0, nblocks, kblocks, lane, row_live, xq, m, k);
    while (true) {
        const int64_t kb1 = kb + step;
        if (kb1 < kblocks)
            gemv_load<NBLK, WAVES, U, RB, XT>(s1, xrow, packed, kb1, nb0, nblocks, kblocks, lane, row_live, xq, m, k);
        gemv_compute<NBLK, WAVES, U, RB, XT>(s0, acc, kb, kblocks, xb, lane);
        if (kb1 >= kblocks) break;
        const int64_t kb2 = kb1 + step;
        if (kb2 < kblocks)
            gemv_load<NBLK, WAVES, U, RB, XT>(s0, xrow, packed, kb2, nb0, nblocks, kblocks, lane, row_live, xq, m, k);
        gemv_compute<NBLK, WAVES, U, RB, XT>(s1, acc, kb1, kblocks, xb, lane);
        if (kb2 >= kblocks) break;
        kb = kb2;
    }
    }

#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int j = 0; j < NBLK; j++) red[wave][b * NBLK + j][lane] = acc[b][j];
    __syncthreads();
    const float g = OUT == OUT_I32 ? 0.0f : (float)gamma[0];  // gamma may be NULL for int32 output
    for (int e = wave; e < RB * NBLK; e += WAVES) {
        const int b = e / NBLK, j = e % NBLK;
        const int64_t nb = nb0 + j;
        if (nb >= nblocks) continue;
        v4i s = red[0][e][lane];
#pragma unroll
        for (int w = 1; w < WAVES; w++) s += red[w][e][lane];
        const int64_t col = nb * 16 + fr;
        const float cb = (OUT != OUT_I32 && bias) ? bias[col] : 0.0f;
        int32_t rs[4];
        float pt[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            if constexpr (RB == 1) {
                rs[r] = rsr[r];
                pt[r] = ptr[r];
            } else {
                const int64_t row = 16 * b + 4 * (lane / 16) + r < m ? 16 * b + 4 * (lane / 16) + r : m - 1;
                rs[r] = rowsum[row];
                pt[r] = OUT == OUT_I32 ? 0.0f : pts[row];
            }
        }
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int64_t row = 16 * b + 4 * (lane / 16) + r;
            if (row < m) epilogue_store<OUT>(out, row * n + col, s[r], rs[r], pt[r], g, bias, cb);
        }
    }
}

template <int NBLK, int WAVES, int U, int RB, int OUT, bool XT = false>
hipError_t launch_gemv(const int8_t *xq, const float *pts, const int32_t *rowsum, const uint32_t *packed,
                       const double *gamma, const float *bias, int64_t m, int64_t n, int64_t k, void *out,
                       hipStream_t st) {
    const int64_t nblocks = n / 16;
    const unsigned grid = (unsigned)((nblocks + NBLK - 1) / NBLK);
    hipLaunchKernelGGL((w2a8_gemv_kernel<NBLK, WAVES, U, RB, OUT, XT>), dim3(grid), dim3(WAVES * 64), 0, st, xq,
                       pts, rowsum, packed, gamma, bias, m, n, k, out);
    return hipGetLastError();
}

// 16 < m <= 64: two to four 16-row blocks.  Every column block a workgroup
// owns re-reads x, so wide products give each workgroup several.  Measured
// on MI355X with the weights streamed from HBM (HIP-graph replays rotating
// copies) at n x k = 4096 x 4096, 11008 x 4096 and 28672 x 8192, m = 17, 32,
// 48, 64, against 1-4 column blocks with 8 waves and 4 with 4 waves: one
// column block up to 384 column blocks, three up to 1024, four with 4 waves
// above (whose larger register budget holds four row blocks' stages).
template <int RB, int OUT>
hipError_t launch_gemv_rows(const int8_t *xq, const float *pts, const int32_t *rowsum, const uint32_t *packed,
                            const double *gamma, const float *bias, int64_t m, int64_t n, int64_t k, void *out,
                            hipStream_t st) {
    const int64_t nblocks = n / 16;
    // x through LDS in whole lines once every wave has k blocks to stream
    // (k >= 2048; at k = 256 the LDS round trip only adds latency); four row
    // blocks of three column blocks have no registers left for it.
    if (k >= 2048) {
        if (nblocks <= 384)
            return launch_gemv<1, 8, 1, RB, OUT, true>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
        if (nblocks <= 1024)
            return launch_gemv<3, 8, 1, RB, OUT, (RB < 4)>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
        return launch_gemv<4, 4, 1, RB, OUT, true>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
    }
    if (nblocks <= 384) return launch_gemv<1, 8, 1, RB, OUT>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
    if (nblocks <= 1024) return launch_gemv<3, 8, 1, RB, OUT>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
    return launch_gemv<4, 4, 1, RB, OUT>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
}

template <int OUT>
hipError_t launch_out(const int8_t *xq, const float *pts, const int32_t *rowsum, const uint32_t *packed,
                      const double *gamma, const float *bias, int64_t m, int64_t n, int64_t k, void *out,
                      hipStream_t st) {
    if (m > 16 && m <= 64) {
        switch ((m + 15) / 16) {
            case 2: return launch_gemv_rows<2, OUT>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
            case 3: return launch_gemv_rows<3, OUT>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
            default: return launch_gemv_rows<4, OUT>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
        }
    }
    if (m > 96 && m <= 128 && k >= 2048 && n / 16 <= 768) {
        // Eight row blocks do not fit the decode kernel's registers; two
        // decode launches of 64 and m - 64 rows (each streaming the weights
        // once) beat the 128 x 256 tiles while each launch's grid fits one
        // round on the CUs (three column blocks per workgroup up to 768
        // column blocks).  Measured at m = 112, k = 2048 / 4096 / 8192: n =
        // 11008 13.9 / 20.5 / 34.0 us against 18.6 / 28.9 / 50.1 on the
        // tiles; n = 16384 24.9 / 37.6 / 64.2 against 18.7 / 29.2 / 50.5.
        const hipError_t e = launch_out<OUT>(xq, pts, rowsum, packed, gamma, bias, 64, n, k, out, st);
        if (e != hipSuccess) return e;
        const int64_t es = OUT == OUT_I32 || OUT == OUT_F32 ? 4 : 2;   // output element bytes
        return launch_out<OUT>(xq + 64 * k, pts ? pts + 64 : nullptr, rowsum + 64, packed, gamma, bias, m - 64, n, k,
                               static_cast<int8_t *>(out) + 64 * n * es, st);
    }
    if (m > 64 && m <= 96 && k >= 2048 && n / 16 <= 1024) {
        // Five or six row blocks: four waves (their register budget holds the
        // stages), two column blocks per workgroup, x through LDS.  Eight row
        // blocks spill even with one column block.  Wider products (x
        // re-read for every two column blocks) stay on the tiles, although
        // at m = 80 the decode kernel still led at 1024 column blocks (16.0
        // against 18.6 us at k = 2048, 37.7-38.1 against 50.3 at k = 8192).
        return launch_gemv<2, 4, 1, 6, OUT, true>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
    }
    if (m <= 16) {
        // Measured on MI355X at k=8192, n=28672 with the weights streamed from
        // HBM, 8 waves and one k block per register stage: 4 column blocks per
        // workgroup up to m = 4, 7 above (1792 column blocks = 256 workgroups).
        // Above m = 4 (and k >= 2048, as for more row blocks), x moves in
        // whole cache lines through LDS, and up to k = 8192 every k block of
        // a wave is loaded at the start (one stage: 13.7-13.9 against
        // 14.6-14.7 us at m = 16; slower at m = 1 and 4 with 7 column blocks).
        if (m <= 4) return launch_gemv<4, 8, 1, 1, OUT>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
        if (k >= 2048 && k / 256 <= 8 * 4)
            return launch_gemv<7, 8, 4, 1, OUT, true>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
        if (k >= 2048)
            return launch_gemv<7, 8, 1, 1, OUT, true>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
        return launch_gemv<7, 8, 1, 1, OUT>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
    }
    // Everything else above 64 rows: the large tiles, also for 64 < m < 256
    // (one or two tile rows), where they beat 128 x 128 tiles on four waves
    // at every measured shape.
    const int64_t tiles_m = (m + XBM - 1) / XBM, tiles_n = (n + XBN - 1) / XBN;
    if (tiles_m * tiles_n > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((w2a8_big_kernel<OUT>), dim3((unsigned)(tiles_m * tiles_n)), dim3(kPThreads), 0, st, xq, pts,
                       rowsum, packed, gamma, bias, m, n, k, out, (int)tiles_m, (int)tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_w2a8(const int8_t *xq, const float *pts, const int32_t *rowsum,
                            const uint32_t *packed, const double *gamma, const float *bias, int64_t m,
                            int64_t n, int64_t k, int out_kind, void *out, hipStream_t st) {
    switch (out_kind) {
        case OUT_F16: return launch_out<OUT_F16>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
        case OUT_BF16: return launch_out<OUT_BF16>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
        default: return launch_out<OUT_I32>(xq, pts, rowsum, packed, gamma, bias, m, n, k, out, st);
    }
}

}  // namespace ql
