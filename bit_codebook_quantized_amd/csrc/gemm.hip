// w4a8_gemm: prefill product for any M on the int8 matrix cores of gfx950.
//
// ai-toolkit convrot_w4a8_quant.py, _w4a8_linear_ste_op: the int8 grid of the
// weight (decoded from 4-bit codes, fp8 group scales and the codebook) times the
// int8 activation rows, accumulated exactly in int32, then the epilogue
// fp32(acc) * (xs[m] * ws[n]) [+ bias[n]].  Unlike the page, which writes the
// decoded int8 weight to memory and runs a library int8 GEMM on it, the weight is
// decoded tile by tile into LDS here, so no int8 weight copy ever reaches HBM.
//
// Tiling.  A block of 512 threads (8 waves, two per SIMD) computes a 256 x 128 output
// tile in stages of 128 k.  Wave w owns rows 64 (w / 2) .. + 63 and columns 64 (w % 2)
// .. + 63: 4 x 4 accumulators of v_mfma_i32_16x16x64_i8, both operands read from LDS.
//
// Memory paths (all full 128-byte lines; 16-row x 64-byte patterns run at well under half
// the L2-to-CU rate):
//  - Activations go straight from global memory into LDS (global_load_lds_dwordx4): 32
//    loads of 8 rows x 128 bytes per stage, no registers or vector instructions.  The
//    16-byte chunks of a 128-byte row are XOR-swizzled by the row pair, so the MFMA
//    fragment reads (16 rows, one chunk each) hit 16 distinct bank groups.
//  - Packed codes come in two stages at a time, one load per stage (16 rows x 64 bytes):
//    lane l takes 16 bytes = two 16-column groups of a fixed row, so its piece of each stage
//    sits in a fixed register and needs no selection.  Each piece is decoded with byte permutes against the LDS level-table row of its
//    group's scale byte and written as two 16-byte fragments into the stage's weight
//    buffer (same swizzle).
//  - Pipeline: three activation buffers and three weight buffers.  Stage s multiplies
//    buffer s % 3; the activations of s + 3 are requested and the weights of s + 2 are
//    decoded meanwhile (half per MFMA half, interleaved with the MFMAs), and the codes of
//    period (s + 4) / 2 are requested on even stages.  One barrier per stage, between the
//    two MFMA halves: after it the first-half fragments of s + 1 are read while the
//    second-half MFMAs of s run.  Steady stages run twelve at a time (the period of the
//    three buffers and the two code slots), so their LDS offsets are constants.
//  - Every vector-memory instruction of the main loop is written as inline asm, so the
//    compiler does not insert waits of its own; each wait below counts the instructions
//    issued after the one it needs (vmcnt retires in issue order).  Code registers are
//    passed through an empty asm after their wait, so no use can move above it.
// MFMA operands are swapped (the weight fragment is the first operand) so that each lane
// ends with 4 consecutive output columns of one row.
//
// Tiles are mapped to blocks so that each of the 8 XCDs (blocks are dealt to XCDs round
// robin) works on a contiguous range of tile ids, and ids run over bands of 4 row tiles
// (row tile fastest), so an XCD's range is a compact block of row x column tiles that
// share activation and weight panels in its L2.
#include <type_traits>

#include "w4a8_device.hpp"

namespace w4a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int GM_THREADS = 512;
constexpr int WM = 4, WN = 2, NW = WM * WN;          // wave grid
constexpr int BM = 256, BN = 128, BK = 128;          // block tile, k per stage
constexpr int TM = BM / WM, TN = BN / WN, MT = TM / 16, NB = TN / 16;
constexpr int A_STAGE = BM * BK;                     // 32 KiB of activations per stage
constexpr int B_STAGE = BN * BK;                     // 16 KiB of decoded weights per stage
constexpr int NBUF = 3;
constexpr int AI = A_STAGE / 1024 / NW;              // activation loads per wave per stage
constexpr int CI = 2 * BN * 128 / 1024 / NW / 2;     // code loads per wave per period (2 stages)
constexpr int CV = 2 * CI;                           // + one scale load each
static_assert(CI == 2, "one code piece per lane and stage");

// position of 16-byte chunk c (0..7) of 128-byte row r
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// The direct-to-LDS load takes its LDS address in m0.  The compiler reserves m0 but uses it
// in none of these kernels (nothing else here needs it on gfx950: no LDS-to-register ops,
// GWS or relative register indexing), so the asm sets it before each load.
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const int8_t*)p);
}
// 64 lanes x 16 bytes from sbase + voff into LDS at m0 + 16 * lane
__device__ __forceinline__ void load_lds16(uint32_t voff, const void* sbase, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, %2" ::"v"(voff), "s"(m0), "s"(sbase)
                 : "memory", "m0");
}
__device__ __forceinline__ v4u load16(uint32_t voff, const void* sbase) {
    v4u x;
    asm volatile("global_load_dwordx4 %0, %1, %2" : "=v"(x) : "v"(voff), "s"(sbase));
    return x;
}
__device__ __forceinline__ uint32_t load_u16(uint32_t voff, const void* sbase) {
    uint32_t x;
    asm volatile("global_load_ushort %0, %1, %2" : "=v"(x) : "v"(voff), "s"(sbase));
    return x;
}
template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N));
}
// at most N vector-memory instructions outstanding and all LDS operations done, then the
// workgroup barrier (the memory clobber keeps LDS accesses on their side of it)
template <int N>
__device__ __forceinline__ void bar_wait() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// the same for a uniform run-time count (only near the ends of the K loop); an unlisted
// count waits for everything, which is always safe
#define W4A8_CASES(F)                                                                                \
    F(1) F(2) F(3) F(4) F(5) F(6) F(7) F(8) F(9) F(10) F(11) F(12) F(13) F(14) F(15) F(16) F(17) F(18) \
        F(19) F(20)
__device__ __forceinline__ void vm_wait_n(int n) {
    switch (n) {
#define W4A8_C(v) case v: vm_wait<v>(); break;
        W4A8_CASES(W4A8_C)
#undef W4A8_C
        default: vm_wait<0>(); break;
    }
}
__device__ __forceinline__ void bar_wait_n(int n) {
    switch (n) {
#define W4A8_C(v) case v: bar_wait<v>(); break;
        W4A8_CASES(W4A8_C)
#undef W4A8_C
        default: bar_wait<0>(); break;
    }
}

template <int OUT>
__global__ __launch_bounds__(GM_THREADS) void gemm_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int M, const uint8_t* __restrict__ qp,
    const uint8_t* __restrict__ srel, const float* __restrict__ codebook, const float* __restrict__ ws,
    const float* __restrict__ bias, int N, int K, void* __restrict__ out, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) int8_t smem[NBUF * (A_STAGE + B_STAGE)];
    __shared__ __attribute__((aligned(16))) uint32_t lut[1024];
    __shared__ __attribute__((aligned(16))) float xs_t[BM], ws_t[BN], bias_t[BN];
    int8_t* const As = smem;
    int8_t* const Bs = smem + NBUF * A_STAGE;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t id = opaque_identity_selector();   // the decode's merge selector base
    const int ntiles = tiles_m * tiles_n;
    int pid = blockIdx.x;
    if ((ntiles & 7) == 0) pid = (pid & 7) * (ntiles >> 3) + (pid >> 3);
    const int band = pid / (4 * tiles_n), tm_first = 4 * band;
    const int band_m = min(tiles_m - tm_first, 4), in_band = pid - band * 4 * tiles_n;
    const int tm = tm_first + in_band % band_m, tn = in_band / band_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int NS = K / BK;   // even, because K % 256 == 0
    const int NP = NS / 2;   // 256-deep code periods
    const int KH = K >> 1, G = K >> 4;

    // ---- activation loads: load j of a wave covers rows 8i .. 8i+7 (i = wave + 8j), lane
    // (row 8i + lane/8, position lane%8), which holds chunk position ^ swz.  Rows past M read
    // row M - 1: they only feed accumulators whose outputs are never stored.
    const int8_t* a_base = xq + (int64_t)m0 * K;
    uint32_t a_off[AI];
#pragma unroll
    for (int j = 0; j < AI; ++j) {
        const int r = 8 * (wave + NW * j) + (lane >> 3);
        a_off[j] = (uint32_t)(min(r, M - 1 - m0) * K + 16 * swz(r, lane & 7));
    }
    const uint32_t a_lds = __builtin_amdgcn_readfirstlane(lds_addr(As) + 1024 * wave);
    auto issue_a = [&](int s, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < AI; ++j) load_lds16(a_off[j], a_base + s * BK, a_lds + buf * A_STAGE + 1024 * NW * j);
    };

    // ---- code loads: load t (0/1) of a wave holds stage t of a 256-deep period for weight
    // rows 16 wave .. 16 wave + 15: lane l takes row 16 wave + l/4 and piece l%4, the 32 codes
    // of groups 2(l%4), 2(l%4)+1 of the stage (16 of the row's 64 bytes), plus the u16 of
    // their two scale bytes.  So a lane's piece of stage t is always code register t and its
    // weight row is fixed.  Rows past N read row N - 1.
    const int crow = 16 * wave + (lane >> 2), cpair = 2 * (lane & 3);
    const uint8_t* q_base = qp + (int64_t)n0 * KH;
    const uint8_t* s_base = srel + (int64_t)n0 * G;
    uint32_t q_off[CI], s_off[CI];
#pragma unroll
    for (int t = 0; t < CI; ++t) {
        const int n = min(crow, N - 1 - n0);
        q_off[t] = (uint32_t)(n * KH + 64 * t + 8 * cpair);
        s_off[t] = (uint32_t)(n * G + 8 * t + cpair);
    }
    struct Codes {
        v4u q[CI];
        uint32_t s[CI];
    };
    auto issue_codes = [&](Codes& c, int period) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < CI; ++jj) {
            c.q[jj] = load16(q_off[jj], q_base + period * 128);
            c.s[jj] = load_u16(s_off[jj], s_base + period * 16);
        }
    };
    // the loads write the code registers asynchronously: after their wait, route the
    // registers through an empty asm so that no use is scheduled before it
    auto tie = [&](Codes& c) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < CI; ++jj) asm volatile("" : "+v"(c.q[jj]), "+v"(c.s[jj]));
    };
    // the lane's piece of stage t (0/1, a constant at every use) of a period: codes and
    // level-table rows
    struct Piece {
        v4u x;
        uint4 t0, t1;
    };
    const uint4* lut4 = reinterpret_cast<const uint4*>(lut);
    auto pick = [&](const Codes& c, int t) __attribute__((always_inline)) {
        Piece p;
        p.x = t ? c.q[1] : c.q[0];
        const uint32_t sc = t ? c.s[1] : c.s[0];
        p.t0 = lut4[sc & 0xFF];
        p.t1 = lut4[(sc >> 8) & 0xFF];
        return p;
    };
    // group g (0/1) of a piece: 16 codes -> 16 int8 levels, one fragment of the weight buffer
    // (row crow, 16-byte chunk cpair + g, swizzled as the activations)
    const int bw[2] = {128 * crow + 16 * swz(crow, cpair), 128 * crow + 16 * swz(crow, cpair + 1)};
    auto decode_group = [&](const Piece& p, int g, int buf) __attribute__((always_inline)) {
        const uint2 d0 = decode8(g ? p.x.z : p.x.x, g ? p.t1 : p.t0, id);
        const uint2 d1 = decode8(g ? p.x.w : p.x.y, g ? p.t1 : p.t0, id);
        *reinterpret_cast<v4u*>(Bs + buf * B_STAGE + bw[g]) = v4u{d0.x, d0.y, d1.x, d1.y};
    };

    // ---- fragments: lane l holds row (or column) l%16 of a 16-row slice, chunk 4h + l/16 of
    // the stage (h = MFMA half); both operands agree on the k order by construction
    int a_rd[MT], b_rd[NB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a_rd[mt] = 128 * (wm * TM + 16 * mt + (lane & 15));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b_rd[nb] = 128 * (wn * TN + 16 * nb + (lane & 15));
    const int rsw = ((lane & 15) >> 1) & 7;   // swz of those rows: their 16-aligned base adds 0
    struct Frag {
        v4i a[MT], b[NB];
    };
    // per half: the lane's offsets of its first A and B fragment (the others follow at 2 KiB
    // steps, within a read instruction's immediate offset)
    const int a_pos[2] = {16 * ((lane >> 4) ^ rsw) + a_rd[0], 16 * ((4 + (lane >> 4)) ^ rsw) + a_rd[0]};
    const int b_pos[2] = {16 * ((lane >> 4) ^ rsw) + b_rd[0], 16 * ((4 + (lane >> 4)) ^ rsw) + b_rd[0]};
    auto read_frags = [&](Frag& f, int buf, int h) __attribute__((always_inline)) {
        const int8_t* ab = As + buf * A_STAGE + a_pos[h];
        const int8_t* bb = Bs + buf * B_STAGE + b_pos[h];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) f.a[mt] = *reinterpret_cast<const v4i*>(ab + 2048 * mt);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) f.b[nb] = *reinterpret_cast<const v4i*>(bb + 2048 * nb);
    };
    v4i acc[MT][NB];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = v4i{0, 0, 0, 0};
    auto mfmas = [&](const Frag& f) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[mt][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.b[nb], f.a[mt], acc[mt][nb], 0, 0, 0);
    };
    // issue order of an MFMA half: each MFMA followed by a share of the fragment reads, the
    // decode's vector instructions and its LDS writes
    auto interleave = [&]() __attribute__((always_inline)) {
        constexpr int NMF = MT * NB, NRD = MT + NB;
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                             // MFMA
            if (i * NRD / NMF != (i + 1) * NRD / NMF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                                             // VALU
            if (i == NMF - 1) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);                          // LDS write
        }
    };

    // ---- epilogue operands (needed after the loop; the compiler waits for them there)
    constexpr int EV = (BM + 2 * BN + GM_THREADS - 1) / GM_THREADS;
    float ev[EV];
    // One unconditional load per value from a clamped address, then a select: loads in
    // separate branches that write the same register would each wait for the previous one.
#pragma unroll
    for (int e = 0; e < EV; ++e) {
        const int i = tid + GM_THREADS * e;
        const bool is_x = i < BM, is_w = !is_x && i < BM + BN, is_b = !is_x && !is_w && i < BM + 2 * BN;
        const int r = is_x ? m0 + i : n0 + (is_w ? i - BM : i - BM - BN);
        const bool ok = is_x ? r < M : (is_w || (is_b && bias)) && r < N;
        const float* src = is_x ? xs : (is_b && bias) ? bias : ws;
        const float v = src[min(r, (is_x ? M : N) - 1)];
        ev[e] = ok ? v : 0.0f;
    }

    // ---- prologue.  Issue order: codes of period 0, A(0), codes of period 1, A(1), A(2)
    // (the first two after the level table is built, the last three after B(0), B(1) are
    // decoded); then
    // stage t issues A(t + 3) and, when t is even, the codes of period (t + 4) / 2.
    // ops_at(t) counts stage t's vector-memory instructions; every wait counts the
    // instructions issued after the one it needs.
    auto ops_at = [&](int t) __attribute__((always_inline)) {
        return (t + 3 < NS ? AI : 0) + ((!(t & 1) && (t + 4) / 2 < NP) ? CV : 0);
    };
    // The codebook (uniform loads) is requested before the tile's loads: behind ~100 KB of
    // loads per CU it would arrive ~2 us later and hold up the level table.
    float cb[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) cb[c] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(codebook[c])));
    // The level table is built first (it waits only for the codebook), then the first
    // period's codes and A(0) go out, and the rest of the prologue's loads follow the decode
    // of B(0), B(1) (the same issue order throughout).
    Codes C0, C1;
    build_level_table_regs(lut, cb, tid, GM_THREADS);
    issue_codes(C0, 0);
    issue_a(0, 0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // level table
    vm_wait<AI>();   // C0 landed (A(0) may still be in flight)
    tie(C0);
    {
        const Piece p0 = pick(C0, 0);
        decode_group(p0, 0, 0);
        decode_group(p0, 1, 0);
        if (NS > 1) {
            const Piece p1 = pick(C0, 1);
            decode_group(p1, 0, 1);
            decode_group(p1, 1, 1);
        }
    }
    if (NP > 1) issue_codes(C1, 1);
    if (NS > 1) issue_a(1, 1);
    if (NS > 2) issue_a(2, 2);
    const int after_a1 = NS > 2 ? AI : 0;
    const int after_p1 = (NS > 1 ? AI : 0) + after_a1;
    const int after_a0 = (NP > 1 ? CV : 0) + after_p1;
    Piece pc;   // the piece of B(s + 2) during stage s
    if (NS > 2) {
        vm_wait_n(after_p1);
        tie(C1);
        pc = pick(C1, 0);
    }
    bar_wait_n(after_a0);   // B(0), B(1) written, A(0) landed
    Frag F0, F1;
    read_frags(F0, 0, 0);

    int buf = 0;   // s % 3
    // steady: 4 <= s <= NS - 5, where every stage around s issues all its loads, so the wait
    // counts are constants
    // par = (s + 1) & 1, a constant at every call; buf_c is the stage's buffer s % 3 when the
    // caller knows it as a constant (then every LDS offset of the stage is a constant too),
    // else -1 and the running `buf` is used
    auto stage = [&](int s, Codes& nxt, Codes& ld, auto steady_c, int par, auto buf_c) __attribute__((always_inline)) {
        constexpr bool steady = decltype(steady_c)::value;
        constexpr int BC = decltype(buf_c)::value;
        const int cb = BC >= 0 ? BC : buf;
        const bool even = par != 0;   // s is even
        const int nbuf = cb == 2 ? 0 : cb + 1, dbuf = nbuf == 2 ? 0 : nbuf + 1;
        const bool dec_on = steady || s + 2 < NS;
        // first half: MFMAs of s, second-half fragments of s, first group of B(s + 2)
        mfmas(F0);
        read_frags(F1, cb, 1);
        if (dec_on) decode_group(pc, 0, dbuf);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        // B(s + 1) complete, A(s + 1) landed (issued at stage s - 2), F1(s) read by every wave
        if (steady) {
            bar_wait<AI + CV>();
        } else {
            int after = 0;
            if (s + 1 < NS) {
                if (s == 0) after = after_a1;
                else if (s == 1) after = ops_at(0);
                else after = ((!(s & 1) && (s + 2) / 2 < NP) ? CV : 0) + ops_at(s - 1);
            }
            bar_wait_n(after);
        }
        if (steady || s + 3 < NS) issue_a(s + 3, cb);
        if (even && (steady || (s + 4) / 2 < NP)) issue_codes(ld, (s + 4) / 2);
        // second half: MFMAs of s, first-half fragments of s + 1, second group of B(s + 2)
        mfmas(F1);
        if (steady || s + 1 < NS) read_frags(F0, nbuf, 0);
        if (dec_on) decode_group(pc, 1, dbuf);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        // the piece of B(s + 3): period (s + 3) / 2, issued at stage 2P - 4 (P >= 2) or in the
        // prologue before A(1) and A(2) (P = 1)
        if (steady || s + 3 < NS) {
            if (steady) {
                if (!even) vm_wait<AI>();
                else vm_wait<2 * AI + CV>();
            } else {
                const int P = (s + 3) / 2;
                int after = P == 1 ? after_p1 : 0;
                for (int t = P == 1 ? 0 : 2 * P - 3; t <= s; ++t) after += ops_at(t);
                vm_wait_n(after);
            }
            tie(nxt);
            pc = pick(nxt, par);   // (s + 1) & 1
        }
        buf = nbuf;
    };
    using Dyn = std::integral_constant<bool, false>;
    using Std = std::integral_constant<bool, true>;
    using BD = std::integral_constant<int, -1>;
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using B2 = std::integral_constant<int, 2>;
    // period P lives in code slot P % 2 (C0 / C1): stage s picks from period (s + 3) / 2 and
    // even stages load period (s + 4) / 2
    auto quad = [&](int s, auto steady_c) __attribute__((always_inline)) {
        stage(s + 0, C1, C0, steady_c, 1, BD{});
        stage(s + 1, C0, C0, steady_c, 0, BD{});
        stage(s + 2, C0, C1, steady_c, 1, BD{});
        stage(s + 3, C1, C1, steady_c, 0, BD{});
    };
    // twelve steady stages from s = 4 (mod 12): the buffers (s % 3) and code slots are constants
    auto dozen = [&](int s) __attribute__((always_inline)) {
        stage(s + 0, C1, C0, Std{}, 1, B1{});
        stage(s + 1, C0, C0, Std{}, 0, B2{});
        stage(s + 2, C0, C1, Std{}, 1, B0{});
        stage(s + 3, C1, C1, Std{}, 0, B1{});
        stage(s + 4, C1, C0, Std{}, 1, B2{});
        stage(s + 5, C0, C0, Std{}, 0, B0{});
        stage(s + 6, C0, C1, Std{}, 1, B1{});
        stage(s + 7, C1, C1, Std{}, 0, B2{});
        stage(s + 8, C1, C0, Std{}, 1, B0{});
        stage(s + 9, C0, C0, Std{}, 0, B1{});
        stage(s + 10, C0, C1, Std{}, 1, B2{});
        stage(s + 11, C1, C1, Std{}, 0, B0{});
    };
    int s = 0;
    if (NS >= 4) {
        quad(0, Dyn{});
        s = 4;
    }
    for (; s + 16 <= NS; s += 12) dozen(s);
    for (; s + 8 <= NS; s += 4) quad(s, Std{});
    for (; s + 4 <= NS; s += 4) quad(s, Dyn{});
    if (s < NS) {
        stage(s + 0, C1, C0, Dyn{}, 1, BD{});
        stage(s + 1, C0, C0, Dyn{}, 0, BD{});
    }

    // ---- epilogue.  Every wave is past the loop's last barrier (no LDS reads remain) and
    // every load of the loop has completed.
#pragma unroll
    for (int e = 0; e < EV; ++e) {
        const int i = tid + GM_THREADS * e;
        if (i < BM) xs_t[i] = ev[e];
        else if (i < BM + BN) ws_t[i - BM] = ev[e];
        else if (i < BM + 2 * BN) bias_t[i - BM - BN] = ev[e];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // accumulator (mt, nb) register r of lane l holds column wn*TN + 16nb + 4(l/16) + r of row
    // wm*TM + 16mt + l%16
    const bool whole = m0 + BM <= M && n0 + BN <= N;
    // bf16 and SwiGLU outputs of a whole tile: each wave passes its 64 x 64 result through its
    // own part of LDS (rows padded by 16 bytes, conflict-free) and stores whole row segments
    // (8 rows x 128 bytes or 16 rows x 64 bytes per instruction) as non-temporal stores
    if ((OUT == 0 || OUT == 3) && whole && (N & 15) == 0) {
        constexpr int OW = OUT == 3 ? TN : 2 * TN;          // output bytes per row of the wave
        constexpr int PITCH = OW + 16;
        uint8_t* ob = reinterpret_cast<uint8_t*>(As) + wave * (TM * PITCH);
        const int rl = lane & 15, cq = lane >> 4;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float xsm = xs_t[wm * TM + 16 * mt + rl];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int nl = 16 * nb + 4 * cq;
                const float4 wv = *reinterpret_cast<const float4*>(&ws_t[wn * TN + nl]);
                const float4 bv = *reinterpret_cast<const float4*>(&bias_t[wn * TN + nl]);
                const v4i a = acc[mt][nb];
                const float wsv[4] = {wv.x, wv.y, wv.z, wv.w}, bsv[4] = {bv.x, bv.y, bv.z, bv.w};
                float y[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    y[r] = __fmul_rn((float)a[r], __fmul_rn(xsm, wsv[r]));
                    if (bias) y[r] = __fadd_rn(y[r], bsv[r]);
                }
                uint8_t* dst = ob + (16 * mt + rl) * PITCH;
                if (OUT == 3) {
                    // gate/up pairs (nl, nl + 1), (nl + 2, nl + 3) -> output columns nl/2, nl/2 + 1
                    *reinterpret_cast<uint32_t*>(dst + nl) =
                        f32x2_to_bf16x2(swiglu_f32(y[0], y[1]), swiglu_f32(y[2], y[3]));
                } else {
                    *reinterpret_cast<uint2*>(dst + 2 * nl) =
                        uint2{f32x2_to_bf16x2(y[0], y[1]), f32x2_to_bf16x2(y[2], y[3])};
                }
            }
        }
        wave_lds_sync();
        constexpr int CPR = OW / 16, RPI = 64 / CPR;   // 16-byte chunks per row, rows per store
        const int64_t row_elems = OUT == 3 ? (N >> 1) : N;
        const int64_t col0 = OUT == 3 ? (n0 + wn * TN) >> 1 : n0 + wn * TN;
#pragma unroll
        for (int i = 0; i < TM / RPI; ++i) {
            const int row = RPI * i + lane / CPR, c = lane % CPR;
            const uint4 v = *reinterpret_cast<const uint4*>(ob + row * PITCH + 16 * c);
            const int64_t m = m0 + wm * TM + row;
            __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w},
                                        reinterpret_cast<v4u*>(reinterpret_cast<uint16_t*>(out) + m * row_elems +
                                                               col0 + 8 * c));
        }
        return;
    }
    const bool vec = whole && (N & 3) == 0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int ml = wm * TM + 16 * mt + (lane & 15), m = m0 + ml;
        if (m >= M) continue;
        const float xsm = xs_t[ml];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int nl = wn * TN + 16 * nb + 4 * (lane >> 4), n = n0 + nl;
            const float4 wv = *reinterpret_cast<const float4*>(&ws_t[nl]);
            const float4 bv = *reinterpret_cast<const float4*>(&bias_t[nl]);
            const v4i a = acc[mt][nb];
            const float wsv[4] = {wv.x, wv.y, wv.z, wv.w}, bsv[4] = {bv.x, bv.y, bv.z, bv.w};
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                y[r] = __fmul_rn((float)a[r], __fmul_rn(xsm, wsv[r]));
                if (bias) y[r] = __fadd_rn(y[r], bsv[r]);
            }
            const int64_t idx = (int64_t)m * N + n;
            if (OUT == 3) {
                // gate/up pairs (n, n + 1) and (n + 2, n + 3) -> columns n/2, n/2 + 1 of [M, N/2]
                uint16_t* o = reinterpret_cast<uint16_t*>(out) + (int64_t)m * (N >> 1) + (n >> 1);
                const uint32_t s01 = f32x2_to_bf16x2(swiglu_f32(y[0], y[1]), swiglu_f32(y[2], y[3]));
                if (vec) {
                    *reinterpret_cast<uint32_t*>(o) = s01;
                } else {
                    if (n + 1 < N) o[0] = (uint16_t)s01;
                    if (n + 3 < N) o[1] = (uint16_t)(s01 >> 16);
                }
            } else if (vec) {
                if (OUT == 0) {
                    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + idx) =
                        uint2{f32x2_to_bf16x2(y[0], y[1]), f32x2_to_bf16x2(y[2], y[3])};
                } else if (OUT == 1) {
                    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + idx) = float4{y[0], y[1], y[2], y[3]};
                } else {
                    *reinterpret_cast<v4i*>(reinterpret_cast<int32_t*>(out) + idx) = a;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N) store_out(out, OUT, idx + r, a[r], y[r]);
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
        hipLaunchKernelGGL(gemm_kernel<0>, g, b, 0, stream, xq, xs, M, qp, srel, codebook, ws, bias, N, K, out,
                           tiles_m, tiles_n);
    else if (out_type == 1)
        hipLaunchKernelGGL(gemm_kernel<1>, g, b, 0, stream, xq, xs, M, qp, srel, codebook, ws, bias, N, K, out,
                           tiles_m, tiles_n);
    else if (out_type == 3)
        hipLaunchKernelGGL(gemm_kernel<3>, g, b, 0, stream, xq, xs, M, qp, srel, codebook, ws, bias, N, K, out,
                           tiles_m, tiles_n);
    else
        hipLaunchKernelGGL(gemm_kernel<2>, g, b, 0, stream, xq, xs, M, qp, srel, codebook, ws, bias, N, K, out,
                           tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace w4a8
