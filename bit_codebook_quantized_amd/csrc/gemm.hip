// w4a8_gemm: prefill product for any M on the int8 matrix cores of gfx950.
//
// ai-toolkit convrot_w4a8_quant.py, _w4a8_linear_ste_op: the int8 grid of the
// weight (decoded from 4-bit codes, fp8 group scales and the codebook) times the
// int8 activation rows, accumulated exactly in int32, then the epilogue
// fp32(acc) * (xs[m] * ws[n]) [+ bias[n]].  Unlike the page, which writes the
// decoded int8 weight to memory and runs a library int8 GEMM on it, the weight is
// decoded tile by tile into LDS here, so no int8 weight copy ever reaches HBM.
//
// Tiling: one block of 512 threads (8 waves) computes a BM x BN = 256 x 128 output
// tile, stepping K by BK = 64.  Per step every thread loads 2 x 16 B of activation
// rows and 8 B of packed codes (one row, one group of 16 columns) plus its scale
// byte, decodes the codes with byte permutes against the LDS level table and
// stores both tiles into LDS.  Tile rows are 64 B = four 16-byte chunks, and chunk c
// of row r sits at position c ^ ((r >> 2) & 3): the writes (4 lanes per row) and the
// fragment reads (16 rows at one chunk) both touch 16 distinct 16-byte bank groups.  The waves
// form a 4 x 2 grid of 64 x 64 sub-tiles, each 4 x 4 v_mfma_i32_16x16x64_i8
// accumulators (64 int32 registers per lane), so two waves fit on each SIMD: the
// LDS only streams fragments near its peak with several waves per SIMD in flight.
// Both MFMA operands are read as 16 consecutive k bytes per lane (lane % 16 = row,
// lane / 16 = which 16-byte quarter of the K-step), so A and B agree on the k order
// by construction.
//
// Tiles are mapped to blocks so that each of the 8 XCDs (blocks are dealt to
// XCDs round robin) works on a contiguous range of tile ids, n fastest, which
// keeps one activation row-panel and neighbouring weight panels in its L2.
#include "w4a8_device.hpp"

namespace w4a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int GM_THREADS = 512;
constexpr int BM = 256, BN = 128, BK = 64;
constexpr int LDSTRIDE = BK;        // bytes per LDS row (64: 4 chunks of 16 B, XOR-swizzled)
constexpr int DEPTH = 4;            // K-steps of global loads in flight
constexpr int NBUF = 3;             // LDS stages: multiply one, fill one two steps ahead

template <int OUT>
__global__ __launch_bounds__(GM_THREADS) void gemm_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int M, const uint8_t* __restrict__ qp,
    const uint8_t* __restrict__ srel, const float* __restrict__ codebook, const float* __restrict__ ws,
    const float* __restrict__ bias, int N, int K, int out_type, void* __restrict__ out, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) uint32_t lut[1024];
    __shared__ __attribute__((aligned(16))) int8_t As[NBUF][BM * LDSTRIDE];
    __shared__ __attribute__((aligned(16))) int8_t Bs[NBUF][BN * LDSTRIDE];
    __shared__ float xs_t[BM], ws_t[BN], bias_t[BN];   // the tile's epilogue scales

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ntiles = tiles_m * tiles_n;
    int pid = blockIdx.x;
    if ((ntiles & 7) == 0) pid = (pid & 7) * (ntiles >> 3) + (pid >> 3);
    const int tn = pid % tiles_n, tm = pid / tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;

    build_level_table(lut, codebook, tid, GM_THREADS);
    const uint4* lut4 = reinterpret_cast<const uint4*>(lut);
    // epilogue operands of this tile, staged once (rows/columns past the edge get 0)
    if (tid < BM) xs_t[tid] = m0 + tid < M ? xs[m0 + tid] : 0.0f;
    if (tid < BN) {
        ws_t[tid] = n0 + tid < N ? ws[n0 + tid] : 0.0f;
        bias_t[tid] = (bias && n0 + tid < N) ? bias[n0 + tid] : 0.0f;
    }

    // global -> register roles
    const int a_row = tid >> 2, a_chk = tid & 3;    // rows a_row and a_row + 128
    // swizzled position of this thread's chunk (a_chk == b_grp; rows a_row, a_row + 128
    // and b_row share (row >> 2) & 3)
    const int w_chunk = (a_chk ^ ((tid >> 4) & 3)) * 16;
    const int b_row = tid >> 2, b_grp = tid & 3;    // one 16-column group of one weight row
    const int KH = K >> 1, G = K >> 4;
    const bool b_ok = n0 + b_row < N;
    const uint8_t* qp_row = qp + (int64_t)(b_ok ? n0 + b_row : 0) * KH + b_grp * 8;
    // the 4 scale bytes of a K-step are one aligned dword; this thread uses byte b_grp
    const uint8_t* sr_row = srel + (int64_t)(b_ok ? n0 + b_row : 0) * G;
    const int s_shift = 8 * b_grp;
    // Rows past M (and columns past N) load row 0: they only feed accumulators whose
    // outputs are never stored, so no masking is needed.
    const int8_t* a_ptr[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int mr = m0 + a_row + 128 * p;
        a_ptr[p] = xq + (int64_t)(mr < M ? mr : 0) * K + a_chk * 16;
    }

    // Register ring of in-flight global loads: slot d holds K-step kt with kt % DEPTH == d.
    // Step kt+1 is written to LDS while step kt is multiplied, and its slot is refilled
    // with step kt+1+DEPTH, so every global load has DEPTH steps of MFMA work to land.
    struct Stage {   // native vector registers only, so the stage lives in VGPRs
        v4u a0, a1;
        v2u b;
        uint32_t s;
    };
    // Loads are unconditional (rows past M or N read row 0, steps past the end re-read
    // the last step) so the count of loads in flight is the same on every path and the
    // compiler can wait for exactly the oldest stage instead of draining all of them.
    auto gload = [&](Stage& st, int kt) __attribute__((always_inline)) {
        const int k0 = kt * BK;
        st.a0 = *reinterpret_cast<const v4u*>(a_ptr[0] + k0);
        st.a1 = *reinterpret_cast<const v4u*>(a_ptr[1] + k0);
        st.b = *reinterpret_cast<const v2u*>(qp_row + (k0 >> 1));
        st.s = *reinterpret_cast<const uint32_t*>(sr_row + (k0 >> 4));
    };
    // Level-table row of a stage's scale byte (one LDS read), then the decode and the
    // LDS writes of the stage; split so the read can be issued well before its use.
    auto lut_row = [&](const Stage& st) __attribute__((always_inline)) {
        return lut4[(st.s >> s_shift) & 0xFFu];
    };
    auto lstore = [&](const Stage& st, const uint4 t, int buf) __attribute__((always_inline)) {
        int8_t* arow = &As[buf][a_row * LDSTRIDE + w_chunk];
        *reinterpret_cast<v4u*>(arow) = st.a0;
        *reinterpret_cast<v4u*>(arow + 128 * LDSTRIDE) = st.a1;
        const uint2 d0 = decode8(st.b.x, t), d1 = decode8(st.b.y, t);
        *reinterpret_cast<v4u*>(&Bs[buf][b_row * LDSTRIDE + w_chunk]) = v4u{d0.x, d0.y, d1.x, d1.y};
    };

    const int wm = wave >> 1, wn = wave & 1;   // 4 x 2 waves of 64 x 64
    v4i acc[4][4];   // [mt][nt] 16 x 16 tiles of the wave's 64 x 64
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int nk = K / BK;   // a multiple of DEPTH because K % 256 == 0
    // v_mfma_i32_16x16x64_i8 operands: lane l holds 16 consecutive k bytes (chunk l / 16 of
    // the K-step's 64) of row (A) or column (B) l % 16; both operands use the same split.
    // rows of a fragment are 16-aligned, so the swizzle term (row >> 2) & 3 is (lane >> 2) & 3
    const int frag_row = lane & 15, frag_k = ((lane >> 4) ^ ((lane >> 2) & 3)) * 16;
    struct Frags {
        v4i a0, a1, a2, a3;   // A rows wm*64 + 16*mt + frag_row
        v4i b0, b1, b2, b3;   // B rows (output columns) wn*64 + 16*nt + frag_row
    };
    auto read_frags = [&](Frags& f, int buf) __attribute__((always_inline)) {
        const int8_t* ab = &As[buf][(wm * 64 + frag_row) * LDSTRIDE + frag_k];
        const int8_t* bb = &Bs[buf][(wn * 64 + frag_row) * LDSTRIDE + frag_k];
        f.a0 = *reinterpret_cast<const v4i*>(ab);
        f.a1 = *reinterpret_cast<const v4i*>(ab + 16 * LDSTRIDE);
        f.a2 = *reinterpret_cast<const v4i*>(ab + 32 * LDSTRIDE);
        f.a3 = *reinterpret_cast<const v4i*>(ab + 48 * LDSTRIDE);
        f.b0 = *reinterpret_cast<const v4i*>(bb);
        f.b1 = *reinterpret_cast<const v4i*>(bb + 16 * LDSTRIDE);
        f.b2 = *reinterpret_cast<const v4i*>(bb + 32 * LDSTRIDE);
        f.b3 = *reinterpret_cast<const v4i*>(bb + 48 * LDSTRIDE);
    };
    auto mfma_step = [&](const Frags& f) __attribute__((always_inline)) {
        const v4i a[4] = {f.a0, f.a1, f.a2, f.a3};
        const v4i b[4] = {f.b0, f.b1, f.b2, f.b3};
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                acc[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
    };

    // Pipeline.  Registers: a ring of four K-steps of global loads (named stages: an
    // indexed private array could be placed in memory by the compiler) and two sets of
    // MFMA fragments.  LDS: three buffers.  Iteration j: barrier (step j+1 is now in LDS
    // for everyone); issue the reads of step j+1's fragments; run step j's MFMAs from the
    // fragments read one iteration earlier, so the LDS reads land while the matrix cores
    // work; decode step j+2 into the third buffer; refill its ring slot with step
    // j+2+DEPTH.
    Stage r0, r1, r2, r3;
    gload(r0, 0);
    gload(r1, min(1, nk - 1));
    gload(r2, min(2, nk - 1));
    gload(r3, min(3, nk - 1));
    __syncthreads();   // level table ready
    lstore(r0, lut_row(r0), 0);
    lstore(r1, lut_row(r1), 1);
    gload(r0, min(4, nk - 1));
    gload(r1, min(5, nk - 1));
    __syncthreads();
    Frags f0, f1;
    read_frags(f0, 0);

    auto step = [&](int j, const Frags& cur, Frags& nxt, Stage& st) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        const uint4 t = lut_row(st);
        read_frags(nxt, (j + 1) % NBUF);   // past the end: reads a buffer nobody uses
        mfma_step(cur);
        lstore(st, t, (j + 2) % NBUF);     // past the end: a harmless write to a buffer nobody reads
        gload(st, min(j + 2 + DEPTH, nk - 1));
        // issue order: the table read, the 8 fragment reads, then the 16 MFMAs each
        // followed by a few decode instructions, then the LDS writes and global loads
        __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int kt0 = 0; kt0 < nk; kt0 += DEPTH) {
        step(kt0 + 0, f0, f1, r2);
        step(kt0 + 1, f1, f0, r3);
        step(kt0 + 2, f0, f1, r0);
        step(kt0 + 3, f1, f0, r1);
    }

    // epilogue: register r of a 16 x 16 accumulator tile holds row 4*(lane/16) + r, column
    // lane % 16; stores of rows past M / columns past N are skipped
    const bool interior = m0 + BM <= M && n0 + BN <= N;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int nl = wn * 64 + nt * 16 + (lane & 15), n = n0 + nl;
        const float wsn = ws_t[nl], bn = bias_t[nl];
        const bool n_ok = n < N;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ml = wm * 64 + mt * 16 + 4 * (lane >> 4) + r, m = m0 + ml;
                const int32_t a = acc[mt][nt][r];
                float y = __fmul_rn((float)a, __fmul_rn(xs_t[ml], wsn));
                if (bias) y = __fadd_rn(y, bn);
                if (interior || (n_ok && m < M)) store_out(out, OUT, (int64_t)m * N + n, a, y);
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const int8_t* xq, const float* xs, int M, const uint8_t* qp, const uint8_t* srel,
                       const float* codebook, const float* ws, const float* bias, int N, int K, int out_type,
                       void* out, hipStream_t stream) {
    (void)hipGetLastError();   // clear a stale error so the check below is about this launch
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int64_t ntiles = (int64_t)tiles_m * tiles_n;
    const dim3 g((unsigned)ntiles), b(GM_THREADS);
    if (out_type == 0)
        hipLaunchKernelGGL(gemm_kernel<0>, g, b, 0, stream, xq, xs, M, qp, srel, codebook, ws, bias, N, K, out_type,
                           out, tiles_m, tiles_n);
    else if (out_type == 1)
        hipLaunchKernelGGL(gemm_kernel<1>, g, b, 0, stream, xq, xs, M, qp, srel, codebook, ws, bias, N, K, out_type,
                           out, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL(gemm_kernel<2>, g, b, 0, stream, xq, xs, M, qp, srel, codebook, ws, bias, N, K, out_type,
                           out, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace w4a8
