// w4a8_gemm: prefill product for any M on the int8 matrix cores of gfx950.
//
// ai-toolkit convrot_w4a8_quant.py, _w4a8_linear_ste_op: the int8 grid of the
// weight (decoded from 4-bit codes, fp8 group scales and the codebook) times the
// int8 activation rows, accumulated exactly in int32, then the epilogue
// fp32(acc) * (xs[m] * ws[n]) [+ bias[n]].  Unlike the page, which writes the
// decoded int8 weight to memory and runs a library int8 GEMM on it, the weight is
// decoded tile by tile into LDS here, so no int8 weight copy ever reaches HBM.
//
// Tiling and roles.  A block of 768 threads computes a 256 x 128 output tile in stages of
// 128 k.  Waves 0..7 (two per SIMD) only multiply: wave w owns rows 64 (w / 2) .. + 63 and
// columns 64 (w % 2) .. + 63, 4 x 4 accumulators of v_mfma_i32_16x16x64_i8, both operands
// read from LDS.  Waves 8..11 (one per SIMD) are producers: they issue every global load
// and decode the weights.  The matrix cores of a SIMD then run beside one wave's vector
// instructions instead of each multiplying wave stopping for its own decode.
//
// Memory paths (all full 128-byte lines or whole 64-byte halves):
//  - Activations go straight from global memory into LDS (global_load_lds_dwordx4): 32
//    loads of 8 rows x 128 bytes per stage, 8 per producer, no registers or vector
//    instructions.  The 16-byte chunks of a 128-byte row are XOR-swizzled by the row pair,
//    so the MFMA fragment reads (16 rows, one chunk each) hit 16 distinct bank groups.
//  - Packed codes come in two stages at a time: producer p owns weight rows 32p .. 32p + 31
//    as two groups of 16, with one load per group and stage (16 rows x 64 bytes): lane l
//    takes 16 bytes = two 16-column groups of a fixed row, so its piece of each stage sits
//    in a fixed register.  Each piece is decoded with byte permutes against the LDS
//    level-table row of its group's scale byte and written as two 16-byte fragments into
//    the stage's weight buffer (same swizzle).
//  - Pipeline: three activation buffers and three weight buffers.  Stage s multiplies
//    buffer s % 3; the producers decode the weights of s + 2 before the stage's barrier,
//    then request the activations of s + 3 and, on even stages, the codes of period
//    (s + 4) / 2.  One barrier per stage, between the two MFMA
//    halves, passed by all 12 waves (each role runs the same sequence of stages, so both
//    pass the same number of barriers): after it the first-half fragments of s + 1 are read
//    while the second-half MFMAs of s run.  Steady stages run twelve at a time (the period
//    of the three buffers and the two code slots), so their LDS offsets are constants.
//  - Every vector-memory instruction of the producers' loop is written as inline asm, so
//    the compiler does not insert waits of its own; each wait counts the instructions the
//    producer issued after the one it needs (vmcnt retires in issue order), and the stage's
//    barrier passes the result on to the multiplying waves.  Code registers are passed
//    through an empty asm after their wait, so no use can move above it.
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

constexpr int NMW = 8, NPW = 4, GM_THREADS = 64 * (NMW + NPW);
constexpr int WM = 4, WN = 2;
constexpr int BM = 256, BN = 128, BK = 128;
constexpr int TM = BM / WM, TN = BN / WN, MT = TM / 16, NB = TN / 16;
constexpr int A_STAGE = BM * BK, B_STAGE = BN * BK, NBUF = 3;
constexpr int AI = A_STAGE / 1024 / NPW;   // activation loads per producer wave per stage (8)
constexpr int CV = 8;                      // code + scale loads per producer wave per period
static_assert(BM + 2 * BN == 64 * NMW, "one epilogue operand (xs, ws or bias) per multiplying thread");
static_assert(BN == 32 * NPW, "each producer owns 32 weight rows of the tile");
static_assert(AI * NPW * 1024 == A_STAGE, "the producers' activation loads cover a stage");

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
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N)); }
// the same for a uniform run-time count (only near the ends of the K loop); an unlisted
// count waits for everything, which is always safe
#define W4A8_CASES(F)                                                                                \
    F(1) F(2) F(3) F(4) F(5) F(6) F(7) F(8) F(9) F(10) F(11) F(12) F(13) F(14) F(15) F(16) F(17) F(18) \
        F(19) F(20) F(21) F(22) F(23) F(24) F(25) F(26) F(27) F(28) F(29) F(30) F(31) F(32) F(33) F(34) F(35) F(36) F(37) F(38) F(39) F(40)
__device__ __forceinline__ void vm_wait_n(int n) {
    switch (n) {
#define W4A8_C(v) case v: vm_wait<v>(); break;
        W4A8_CASES(W4A8_C)
#undef W4A8_C
        default: vm_wait<0>(); break;
    }
}
// the wave's LDS operations done, then the workgroup barrier (the memory clobber keeps LDS
// accesses on their side of it)
__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform, in a scalar register
    const bool prod = wave >= NMW;
    const int ntiles = tiles_m * tiles_n;
    int pid = blockIdx.x;
    if ((ntiles & 7) == 0) pid = (pid & 7) * (ntiles >> 3) + (pid >> 3);
    const int band = pid / (4 * tiles_n), tm_first = 4 * band;
    const int band_m = min(tiles_m - tm_first, 4), in_band = pid - band * 4 * tiles_n;
    const int tm = tm_first + in_band % band_m, tn = in_band / band_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int NS = K / BK, NP = NS / 2, KH = K >> 1, G = K >> 4;

    // epilogue operands: threads 0..511 (the MFMA waves) hold the tile's xs, ws and bias
    float ev = 0.0f;
    if (!prod) {
        const int i = tid;
        const bool is_x = i < BM, is_w = !is_x && i < BM + BN, is_b = !is_x && !is_w;
        const int r = is_x ? m0 + i : n0 + (is_w ? i - BM : i - BM - BN);
        const bool ok = is_x ? r < M : (is_w || (is_b && bias)) && r < N;
        const float* src = is_x ? xs : (is_b && bias) ? bias : ws;
        const float v = src[min(r, (is_x ? M : N) - 1)];
        ev = ok ? v : 0.0f;
    }
    // the level table, built by all 12 waves before any of the tile's loads (it waits only for
    // the codebook, uniform loads)
    float cbv[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) cbv[c] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(codebook[c])));
    build_level_table_regs(lut, cbv, tid, GM_THREADS);

    using Dyn = std::integral_constant<bool, false>;
    using Std = std::integral_constant<bool, true>;
    using BD = std::integral_constant<int, -1>;
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using B2 = std::integral_constant<int, 2>;

    // The stage sequence, the same for both roles (so both pass the same barriers):
    // stage(s, slot of the pieces of B(s+3), slot loaded at even s, steady, par = (s+1)&1, buf)
    auto run_stages = [&](auto stage) __attribute__((always_inline)) {
        auto quad = [&](int s, auto steady_c) __attribute__((always_inline)) {
            stage(s + 0, 1, 0, steady_c, 1, BD{});
            stage(s + 1, 0, 0, steady_c, 0, BD{});
            stage(s + 2, 0, 1, steady_c, 1, BD{});
            stage(s + 3, 1, 1, steady_c, 0, BD{});
        };
        auto dozen = [&](int s) __attribute__((always_inline)) {
            stage(s + 0, 1, 0, Std{}, 1, B1{});
            stage(s + 1, 0, 0, Std{}, 0, B2{});
            stage(s + 2, 0, 1, Std{}, 1, B0{});
            stage(s + 3, 1, 1, Std{}, 0, B1{});
            stage(s + 4, 1, 0, Std{}, 1, B2{});
            stage(s + 5, 0, 0, Std{}, 0, B0{});
            stage(s + 6, 0, 1, Std{}, 1, B1{});
            stage(s + 7, 1, 1, Std{}, 0, B2{});
            stage(s + 8, 1, 0, Std{}, 1, B0{});
            stage(s + 9, 0, 0, Std{}, 0, B1{});
            stage(s + 10, 0, 1, Std{}, 1, B2{});
            stage(s + 11, 1, 1, Std{}, 0, B0{});
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
            stage(s + 0, 1, 0, Dyn{}, 1, BD{});
            stage(s + 1, 0, 0, Dyn{}, 0, BD{});
        }
    };

    if (prod) {
        // ================= producer waves: loads and decode =================
        const int pw = wave - NMW;
        // the producers issue ahead of the multiplying waves on their SIMD (measured: 4% at
        // M = 2048): a stage can start only when they have delivered its operands
        __builtin_amdgcn_s_setprio(2);
        const uint32_t id = opaque_identity_selector();
        const int8_t* a_base = xq + (int64_t)m0 * K;
        uint32_t a_off[AI];
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int r = 8 * (pw + NPW * j) + (lane >> 3);
            a_off[j] = (uint32_t)(min(r, M - 1 - m0) * K + 16 * swz(r, lane & 7));
        }
        const uint32_t a_lds = __builtin_amdgcn_readfirstlane(lds_addr(As) + 1024 * pw);
        auto issue_a = [&](int s, int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < AI; ++j)
                load_lds16(a_off[j], a_base + s * BK, a_lds + buf * A_STAGE + 1024 * NPW * j);
        };
        // codes: row group g (0/1) = rows 32 pw + 16 g .. + 15; load (g, t) holds stage t
        const int cpair = 2 * (lane & 3);
        int crow[2];
        crow[0] = 32 * pw + (lane >> 2);
        crow[1] = crow[0] + 16;
        const uint8_t* q_base = qp + (int64_t)n0 * KH;
        const uint8_t* s_base = srel + (int64_t)n0 * G;
        uint32_t q_off[2], s_off[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int n = min(crow[g], N - 1 - n0);
            q_off[g] = (uint32_t)(n * KH + 8 * cpair);
            s_off[g] = (uint32_t)(n * G + cpair);
        }
        struct Codes {
            v4u q[2][2];
            uint32_t s[2][2];
        };
        auto issue_codes = [&](Codes& c, int period) __attribute__((always_inline)) {
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    c.q[g][t] = load16(q_off[g] + 64 * t, q_base + period * 128);
                    c.s[g][t] = load_u16(s_off[g] + 8 * t, s_base + period * 16);
                }
        };
        auto tie = [&](Codes& c) __attribute__((always_inline)) {
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int t = 0; t < 2; ++t) asm volatile("" : "+v"(c.q[g][t]), "+v"(c.s[g][t]));
        };
        struct Piece {
            v4u x;
            uint4 t0, t1;
        };
        const uint4* lut4 = reinterpret_cast<const uint4*>(lut);
        auto pick = [&](const Codes& c, int g, int t) __attribute__((always_inline)) {
            Piece p;
            p.x = t ? c.q[g][1] : c.q[g][0];
            const uint32_t sc = t ? c.s[g][1] : c.s[g][0];
            p.t0 = lut4[sc & 0xFF];
            p.t1 = lut4[(sc >> 8) & 0xFF];
            return p;
        };
        int bw[2][2];
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int h = 0; h < 2; ++h) bw[g][h] = 128 * crow[g] + 16 * swz(crow[g], cpair + h);
        auto decode_group = [&](const Piece& p, int g, int h, int buf) __attribute__((always_inline)) {
            const uint2 d0 = decode8(h ? p.x.z : p.x.x, h ? p.t1 : p.t0, id);
            const uint2 d1 = decode8(h ? p.x.w : p.x.y, h ? p.t1 : p.t0, id);
            *reinterpret_cast<v4u*>(Bs + buf * B_STAGE + bw[g][h]) = v4u{d0.x, d0.y, d1.x, d1.y};
        };
        auto ops_at = [&](int t) __attribute__((always_inline)) {
            return (t + 3 < NS ? AI : 0) + ((!(t & 1) && (t + 4) / 2 < NP) ? CV : 0);
        };
        Codes C[2];
        issue_codes(C[0], 0);
        issue_a(0, 0);
        barrier();   // level table
        vm_wait<AI>();   // period 0's codes landed
        tie(C[0]);
        {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const Piece p0 = pick(C[0], g, 0);
                decode_group(p0, g, 0, 0);
                decode_group(p0, g, 1, 0);
                if (NS > 1) {
                    const Piece p1 = pick(C[0], g, 1);
                    decode_group(p1, g, 0, 1);
                    decode_group(p1, g, 1, 1);
                }
            }
        }
        if (NP > 1) issue_codes(C[1], 1);
        if (NS > 1) issue_a(1, 1);
        if (NS > 2) issue_a(2, 2);
        const int after_a1 = NS > 2 ? AI : 0;
        const int after_p1 = (NS > 1 ? AI : 0) + after_a1;
        const int after_a0 = (NP > 1 ? CV : 0) + after_p1;
        Piece pc[2];
        if (NS > 2) {
            vm_wait_n(after_p1);
            tie(C[1]);
            pc[0] = pick(C[1], 0, 0);
            pc[1] = pick(C[1], 1, 0);
        }
        vm_wait_n(after_a0);
        barrier();   // B(0), B(1) written, A(0) landed
        int buf = 0;
        run_stages([&](int s, int nxt_slot, int ld_slot, auto steady_c, int par, auto buf_c) __attribute__((always_inline)) {
            constexpr bool steady = decltype(steady_c)::value;
            constexpr int BC = decltype(buf_c)::value;
            const int cb = BC >= 0 ? BC : buf;
            const bool even = par != 0;
            const int nbuf = cb == 2 ? 0 : cb + 1, dbuf = nbuf == 2 ? 0 : nbuf + 1;
            const bool dec_on = steady || s + 2 < NS;
            if (dec_on) {
                decode_group(pc[0], 0, 0, dbuf);
                decode_group(pc[1], 1, 0, dbuf);
                decode_group(pc[0], 0, 1, dbuf);
                decode_group(pc[1], 1, 1, dbuf);
            }
            if (steady) {
                vm_wait<AI + CV>();
            } else {
                int after = 0;
                if (s + 1 < NS) {
                    if (s == 0) after = after_a1;
                    else if (s == 1) after = ops_at(0);
                    else after = ((!(s & 1) && (s + 2) / 2 < NP) ? CV : 0) + ops_at(s - 1);
                }
                vm_wait_n(after);
            }
            barrier();
            if (steady || s + 3 < NS) issue_a(s + 3, cb);
            if (even && (steady || (s + 4) / 2 < NP)) issue_codes(C[ld_slot], (s + 4) / 2);
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
                tie(C[nxt_slot]);
                pc[0] = pick(C[nxt_slot], 0, par);
                pc[1] = pick(C[nxt_slot], 1, par);
            }
            buf = nbuf;
        });
        return;
    }

    // ================= MFMA waves =================
    const int wm = wave / WN, wn = wave % WN;
    int a_rd0 = 128 * (wm * TM + (lane & 15)), b_rd0 = 128 * (wn * TN + (lane & 15));
    const int rsw = ((lane & 15) >> 1) & 7;
    const int a_pos[2] = {16 * ((lane >> 4) ^ rsw) + a_rd0, 16 * ((4 + (lane >> 4)) ^ rsw) + a_rd0};
    const int b_pos[2] = {16 * ((lane >> 4) ^ rsw) + b_rd0, 16 * ((4 + (lane >> 4)) ^ rsw) + b_rd0};
    struct Frag {
        v4i a[MT], b[NB];
    };
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
    auto interleave = [&]() __attribute__((always_inline)) {
        constexpr int NMF = MT * NB, NRD = MT + NB;
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i * NRD / NMF != (i + 1) * NRD / NMF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };
    // the tile's scales go to LDS now (the wait for them costs nothing: these waves wait for
    // the producers' prologue anyway); the loop's barriers publish them
    if (tid < BM) xs_t[tid] = ev;
    else if (tid < BM + BN) ws_t[tid - BM] = ev;
    else bias_t[tid - BM - BN] = ev;
    barrier();   // level table
    barrier();   // B(0), B(1) written, A(0) landed
    Frag F0, F1;
    read_frags(F0, 0, 0);
    int buf = 0;
    run_stages([&](int s, int, int, auto steady_c, int, auto buf_c) __attribute__((always_inline)) {
        constexpr bool steady = decltype(steady_c)::value;
        constexpr int BC = decltype(buf_c)::value;
        const int cb = BC >= 0 ? BC : buf;
        const int nbuf = cb == 2 ? 0 : cb + 1;
        mfmas(F0);
        read_frags(F1, cb, 1);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        barrier();
        mfmas(F1);
        if (steady || s + 1 < NS) read_frags(F0, nbuf, 0);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        buf = nbuf;
    });

    // ---- epilogue (every MFMA wave is past the last stage's barrier: no fragment read of
    // the stage buffers remains, and the producers' loads have all landed)
    // lane-derived values are recomputed from an opaque copy of the lane index, so that the
    // compiler does not keep them in registers (or spill them) through the main loop
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    const bool whole = m0 + BM <= M && n0 + BN <= N;
    if ((OUT == 0 || OUT == 3) && whole && (N & 15) == 0) {
        constexpr int OW = OUT == 3 ? TN : 2 * TN;
        constexpr int PITCH = OW + 16;
        uint8_t* ob = reinterpret_cast<uint8_t*>(As) + wave * (TM * PITCH);
        const int rl = lane_e & 15, cq = lane_e >> 4;
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
                    *reinterpret_cast<uint32_t*>(dst + nl) =
                        f32x2_to_bf16x2(swiglu_f32(y[0], y[1]), swiglu_f32(y[2], y[3]));
                } else {
                    *reinterpret_cast<uint2*>(dst + 2 * nl) =
                        uint2{f32x2_to_bf16x2(y[0], y[1]), f32x2_to_bf16x2(y[2], y[3])};
                }
            }
        }
        wave_lds_sync();
        constexpr int CPR = OW / 16, RPI = 64 / CPR;
        const int64_t row_elems = OUT == 3 ? (N >> 1) : N;
        const int64_t col0 = OUT == 3 ? (n0 + wn * TN) >> 1 : n0 + wn * TN;
#pragma unroll
        for (int i = 0; i < TM / RPI; ++i) {
            const int row = RPI * i + lane_e / CPR, c = lane_e % CPR;
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
        const int ml = wm * TM + 16 * mt + (lane_e & 15), m = m0 + ml;
        if (m >= M) continue;
        const float xsm = xs_t[ml];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int nl = wn * TN + 16 * nb + 4 * (lane_e >> 4), n = n0 + nl;
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
#define W4A8_GEMM_LAUNCH(O)                                                                                   \
    hipLaunchKernelGGL(gemm_kernel<O>, g, b, 0, stream, xq, xs, M, qp, srel, codebook, ws, bias, N, K, out, \
                       tiles_m, tiles_n)
    if (out_type == 0) W4A8_GEMM_LAUNCH(0);
    else if (out_type == 1) W4A8_GEMM_LAUNCH(1);
    else if (out_type == 3) W4A8_GEMM_LAUNCH(3);
    else W4A8_GEMM_LAUNCH(2);
#undef W4A8_GEMM_LAUNCH
    return hipGetLastError();
}

}  // namespace w4a8
