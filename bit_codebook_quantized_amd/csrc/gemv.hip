// w4a8_gemv: decode-path product for M <= 8 token rows, on the vector ALUs.
//
// ai-toolkit convrot_w4a8_quant.py, w4a8_gemv_kernel: the packed codes, the fp8
// group scales and the codebook are read directly, every weight is decoded to its
// int8 grid value in registers and multiply-accumulated in int32 against the int8
// activation rows (exact, so the result equals the matrix-core path bit for bit),
// and the epilogue fp32(acc) * (xs[m] * ws[n]) [+ bias[n]] is fused into the store.
// Weight traffic is 4 bits per code plus one scale byte per 16 codes (4.5 bit per
// weight), which bounds the kernel by HBM bandwidth.
//
// Layout.  A block of 256 threads = 4 waves; wave w owns R consecutive output rows.
// Its 64 lanes split K into 16-column groups (8 bytes of codes + 1 scale byte).  A
// batch covers 64 * NB groups: lane l takes the NB consecutive groups NB*l .. NB*l + NB - 1
// of each row (NB = 4: two 16-byte code loads and one scale dword per row; NB = 3, for K
// a multiple of 3072 and not of 4096: a 16-byte and an 8-byte code load and one 8-byte
// scale load, so that no lane idles when K = 3072).  A batch's weight loads for all R rows
// are issued together and the next batch is prefetched while the current one is decoded.
// The first batch is issued before the block builds its 256 x 16 level table in LDS and
// stages the int8 activations (M x up to 32 KiB, reused by all R rows of all 4 waves) in
// LDS.
//
// Arithmetic per 16-column group and row: one LDS read of the 16-level table row
// of the group's scale byte, two 8-code byte-permute decodes that return even
// columns before odd ones (the activation slab is stored in that order), and 4
// v_dot4_i32_i8 per activation row.  The int32 partial sums of the R x M outputs stay in
// registers for the whole of K and are combined across the wave once, by a
// reduce-scatter (each halving step exchanges half the values), so a lane ends
// with one fully summed output.
#include <atomic>
#include <type_traits>

#include "../../include/w4a8.h"
#include "w4a8_device.hpp"
#include "rotq_device.hpp"

namespace w4a8 {
namespace {

constexpr int GV_THREADS = 256;
constexpr int GEMV_GROUP_MAX = 64;   // layers per grouped launch (the table travels in the kernel arguments)
constexpr int GV_ROUNDS = 4;         // a grouped launch is at most this many rounds of resident blocks

constexpr int pow2_ceil(int v) { return v <= 1 ? 1 : 2 * pow2_ceil((v + 1) / 2); }
constexpr int log2i(int v) { return v <= 1 ? 0 : 1 + log2i(v / 2); }

// Columns of activations held in LDS at a time.
__host__ __device__ constexpr int slab_cols(int mm) { return mm == 1 ? 32768 : mm == 2 ? 16384 : mm <= 4 ? 8192 : 4096; }

// A batch: lane l takes the NB consecutive groups NB*l .. NB*l + NB - 1 of the batch's
// 64*NB of each of its R rows: 8*NB bytes of codes (q[r][2u], q[r][2u + 1] = group u)
// and the NB scale bytes (byte u of s[r]).
template <int R, int NB>
struct Batch {
    uint32_t q[R][2 * NB];
    uint32_t s[R];
    float w[R], b[R];   // the rows' channel scales and biases (epilogue operands)
};

// 16 and 8 bytes at 8-byte (code rows) or 4-byte (scale rows) aligned addresses
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

// Groups per lane and batch for a K-column row whose activations fit one slab: 3 when
// that leaves fewer lanes idle than 4 and K / 16 is a multiple of 3 (a lane's groups
// are then all inside the row or all past it), else 4.
__host__ __device__ constexpr int gemv_nb(int K, int slab) {
    const int g = K >> 4;
    const int idle4 = (g + 255) / 256 * 256 - g, idle3 = (g + 191) / 192 * 192 - g;
    return (K <= slab && g % 3 == 0 && idle3 < idle4) ? 3 : 4;
}

// Loads are unconditional (lanes past the row end re-read its last groups), so the
// compiler can count the loads in flight and wait for exactly the batch it needs.
template <int R, int NB>
__device__ __forceinline__ void load_batch(Batch<R, NB>& b, const uint8_t* const (&qrow)[R], const uint8_t* const (&srow)[R],
                                           int jbase, int nchunk) {
    const int j = min(jbase, nchunk - NB);   // nchunk is a multiple of 16 (and of 3 for NB = 3)
    if constexpr (NB == 4) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint4 lo = *reinterpret_cast<const uint4*>(qrow[r] + (int64_t)j * 8);
            const uint4 hi = *reinterpret_cast<const uint4*>(qrow[r] + (int64_t)j * 8 + 16);
            b.q[r][0] = lo.x; b.q[r][1] = lo.y; b.q[r][2] = lo.z; b.q[r][3] = lo.w;
            b.q[r][4] = hi.x; b.q[r][5] = hi.y; b.q[r][6] = hi.z; b.q[r][7] = hi.w;
            b.s[r] = *reinterpret_cast<const uint32_t*>(srow[r] + j);
        }
    } else {
        // the 3 scale bytes j .. j + 2 from the 8 bytes at the dword below j, moved back to
        // stay inside the row (nchunk - 8 <= j4 <= j, j - j4 <= 5)
        const int j4 = min(j & ~3, nchunk - 8), sh = 8 * (j - j4);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32x4_a4 lo = *reinterpret_cast<const u32x4_a4*>(qrow[r] + (int64_t)j * 8);
            const u32x2_a4 hi = *reinterpret_cast<const u32x2_a4*>(qrow[r] + (int64_t)j * 8 + 16);
            b.q[r][0] = lo.x; b.q[r][1] = lo.y; b.q[r][2] = lo.z; b.q[r][3] = lo.w;
            b.q[r][4] = hi.x; b.q[r][5] = hi.y;
            const u32x2_a4 sv = *reinterpret_cast<const u32x2_a4*>(srow[r] + j4);
            b.s[r] = (uint32_t)((((uint64_t)sv.y << 32) | sv.x) >> sh);
        }
    }
}

// Position of 16-byte chunk c of an activation slab in LDS.  NB = 4: the two low bits
// are XORed with bits 4-5, so the 16 lanes of a read (chunks 4l + u, l = 0..15) hit 16
// different bank groups.  NB = 3: unchanged (chunks 3l + u of 16 consecutive lanes are
// already 16 different ones modulo 16).
template <int NB>
__device__ __forceinline__ int act_chunk(int c) { return NB == 4 ? c ^ ((c >> 4) & 3) : c; }

// Inside a chunk each 8-column half is stored even columns first: bytes k0 k2 k4 k6 k1 k3
// k5 k7, the order in which decode_split returns the weights, so the products need no
// re-interleave of the decoded bytes.
__device__ __forceinline__ uint4 act_split(uint4 v) {
    return uint4{perm(v.y, v.x, 0x06040200u), perm(v.y, v.x, 0x07050301u), perm(v.w, v.z, 0x06040200u),
                 perm(v.w, v.z, 0x07050301u)};
}
__device__ __forceinline__ uint4 act_merge(uint4 v) {   // inverse of act_split
    return uint4{perm(v.y, v.x, 0x05010400u), perm(v.y, v.x, 0x07030602u), perm(v.w, v.z, 0x05010400u),
                 perm(v.w, v.z, 0x07030602u)};
}
// byte position of column j (0..15) of a chunk
__device__ __forceinline__ int act_byte(int j) { return (j & 8) | ((j & 1) << 2) | ((j >> 1) & 3); }


// The value of lane l ^ o (o a power of two, every lane active) without going through
// LDS where gfx950 has a register path: the permlane swaps for 32 and 16 (each returns
// this lane's value and its partner's, in an order set by the lane's half or row
// parity), DPP for 8 (row rotate) and for 2 and 1 (quad permutes); 4 takes a swizzle.
__device__ __forceinline__ int32_t lane_xor(int32_t v, int o, int lane) {
    if (o == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
        return (int32_t)(lane < 32 ? r[1] : r[0]);
    }
    if (o == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
        return (int32_t)((lane & 16) ? r[0] : r[1]);
    }
    if (o == 8) return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);   // row_ror:8
    if (o == 4) return __builtin_amdgcn_ds_swizzle(v, 0x101F);                      // xor 4 in 32 lanes
    if (o == 2) return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);    // quad [2, 3, 0, 1]
    return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);                // quad [1, 0, 3, 2]
}

// Activation staging: MM rows x cols bytes of xq from column k0 (cols <= slab_cols(MM))
// -> act[m * slab_cols(MM) ...].  Every load is issued before the first wait; `between`
// runs after the loads and before the stores (the GEMV issues its first weight batch
// there).  NC uint4 per thread and row, a compile-time count (an index guarded by a
// run-time test would keep the staging registers in scratch memory): chunks past the row
// end are clamped to its last chunk and rewrite it with the same bytes.
template <int MM, int NB, int NC, typename F>
__device__ __forceinline__ void stage_acts_n(uint8_t* act, const int8_t* __restrict__ xq, int K, int k0, int per_row,
                                             int tid, F&& between) {
    uint4 v[MM][NC];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int i = min(tid + 256 * c, per_row - 1);
            v[m][c] = *reinterpret_cast<const uint4*>(xq + (int64_t)m * K + k0 + i * 16);
        }
    between();
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int i = min(tid + 256 * c, per_row - 1);
            *reinterpret_cast<uint4*>(act + m * slab_cols(MM) + act_chunk<NB>(i) * 16) = act_split(v[m][c]);
        }
}

template <int MM, int NB, typename F>
__device__ __forceinline__ void stage_acts(uint8_t* act, const int8_t* __restrict__ xq, int K, int k0, int cols,
                                           int tid, F&& between) {
    constexpr int PER = slab_cols(MM) / 16 / 256;   // at most 8
    const int per_row = cols >> 4;
    if (per_row <= 256 || PER == 1) stage_acts_n<MM, NB, 1>(act, xq, K, k0, per_row, tid, between);
    else if (per_row <= 512 || PER == 2) stage_acts_n<MM, NB, (PER < 2 ? PER : 2)>(act, xq, K, k0, per_row, tid, between);
    else if (per_row <= 1024 || PER == 4) stage_acts_n<MM, NB, (PER < 4 ? PER : 4)>(act, xq, K, k0, per_row, tid, between);
    else stage_acts_n<MM, NB, PER>(act, xq, K, k0, per_row, tid, between);
}

// Bytes of dynamic LDS of a GEMV block: level table, activation slab, the rows' scales,
// and for the fused form the rotation's transpose buffer and the row maxima.
__host__ __device__ constexpr size_t gemv_lds_bytes(int mm, bool fused) {
    return 4096 + (size_t)mm * slab_cols(mm) + 32 + (fused ? ROTQ_TBUF_DOUBLES * 8 + 2 * 16 * 4 : 0);
}

// The fused form's activation preparation: the block rotates and quantises the MM bf16
// rows itself (K <= slab_cols(MM)), with the arithmetic of rotate_quant_act, into the
// activation slab and the scale slots.  Slot s of 16 lanes rotates the 256-column blocks
// s, s + 16, ... of a row; the row maximum is taken over the 16 slots.  The work is a
// sequence of jobs, one 256-column block per slot each: one job per row when K <= 4096
// (the rotated values stay in registers between the maximum and the quantisation), else
// nch jobs for the maximum and nch jobs that rotate again and quantise.  The inputs of
// job j + 2 are loaded while jobs j and j + 1 are computed (two named buffers, so no
// register copy of a load in flight).  `first` holds the inputs of jobs 0 and 1, loaded
// by the caller (rot_first_job) before anything else.  xq_out /
// xs_out, when not null, receive the same int8 rows and scales.
// job j's block for this lane's slot, clamped into range (out-of-range slots are zeroed)
__device__ __forceinline__ RotIn rot_job_load(const uint16_t* __restrict__ x, int K, int j, int njobs,
                                              int jobs_per_row, int nch) {
    j = min(j, njobs - 1);   // past the end: a harmless reload of the last job
    const int row = j / jobs_per_row, c = j - row * jobs_per_row;
    const int blk = min((int)(threadIdx.x >> 4) + 16 * (c % nch), (K >> 8) - 1);
    return rot_load(x, row, K, blk, threadIdx.x & 15);
}

__device__ __forceinline__ int rot_jobs_per_row(int K) {
    const int nch = ((K >> 8) + 15) >> 4;
    return nch == 1 ? 1 : 2 * nch;
}

template <int MM>
__device__ __forceinline__ RotIn rot_first_job(const uint16_t* __restrict__ x, int K, int j) {
    const int nch = ((K >> 8) + 15) >> 4, jpr = rot_jobs_per_row(K);
    return rot_job_load(x, K, j, MM * jpr, jpr, nch);
}

template <int MM, int NB, bool LONGK>
__device__ __forceinline__ void rotate_quant_to_lds(uint8_t* act, float* xs_lds, double* tbuf, float* smax,
                                                    const uint16_t* __restrict__ x, int K, int qmax,
                                                    const RotIn first0, const RotIn first1,
                                                    int8_t* __restrict__ xq_out,
                                                    float* __restrict__ xs_out) {
    constexpr int SLAB = slab_cols(MM);
    const int tid = threadIdx.x, slot = tid >> 4, l16 = tid & 15;
    const int nb = K >> 8, nch = LONGK ? (nb + 15) >> 4 : 1;   // LONGK: K > 4096
    const int jobs_per_row = LONGK ? rot_jobs_per_row(K) : 1;
    const int njobs = MM * jobs_per_row;
    const float qmaxf = (float)qmax;
    float r[16];
    float amax = 0.0f, scale = 1.0f;
    bool poisoned = false;
    double inv = 1.0;

    auto load_job = [&](int j) __attribute__((always_inline)) {
        return rot_job_load(x, K, j, njobs, jobs_per_row, nch);
    };
    auto run_job = [&](int j, const RotIn in) __attribute__((always_inline)) {
        const int row = j / jobs_per_row, c = j - row * jobs_per_row;
        const bool pass1 = nch == 1 || c < nch;
        const int cc = nch == 1 ? 0 : (pass1 ? c : c - nch);
        const int blk = slot + 16 * cc;
        const bool ok = blk < nb;
        rotate_loaded<true>(in, ok, slot, l16, tbuf, r);   // exchanges within each slot's wave
        if (pass1) {
            if (cc == 0) amax = 0.0f;
            amax = block_absmax(r, amax);
            if (cc == nch - 1) {
                const float a = slot_max(amax);
                // alternate rows: every thread reads row r's maxima before it reaches row r + 1's
                // barrier, and row r + 2 writes only after that barrier
                float* sm = smax + 16 * (row & 1);
                if (l16 == 0) sm[slot] = a;
                __syncthreads();
                float rmax = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) rmax = __builtin_fmaxf(rmax, sm[i]);
                scale = row_scale(rmax, qmaxf);
                poisoned = row_poisoned(rmax);   // block-uniform: the block holds one row
                inv = poisoned ? 0.0 : 1.0 / (double)scale;
                if (tid == 0) {
                    xs_lds[row] = scale;
                    if (xs_out) xs_out[row] = scale;
                }
            }
        }
        if ((nch == 1 || !pass1) && ok) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                act[row * SLAB + act_chunk<NB>(16 * blk + i) * 16 + act_byte(l16)] =
                    poisoned ? (uint8_t)0 : quant1(r[i], inv, qmaxf);
        }
    };

    RotIn bA = first0, bB = first1;
    if constexpr (!LONGK) {
        // K <= 4096, one job per row: straight-line code (exact wait counts for the loads
        // in flight; a kernel holds only one of the two forms, so no merged wait state)
#pragma unroll
        for (int j = 0; j < MM; j += 2) {
            run_job(j, bA);
            if (j + 2 < MM) bA = load_job(j + 2);
            if (j + 1 < MM) {
                run_job(j + 1, bB);
                if (j + 3 < MM) bB = load_job(j + 3);
            }
        }
    } else {
        for (int j = 0; j < njobs; j += 2) {
            run_job(j, bA);
            bA = load_job(j + 2);
            if (j + 1 < njobs) run_job(j + 1, bB);
            bB = load_job(j + 3);
        }
    }
    if (xq_out) {   // block-uniform
        __syncthreads();
        const int per_row = K >> 4;
        for (int i = tid; i < MM * per_row; i += GV_THREADS) {
            const int m = i / per_row, c = i - m * per_row;
            *reinterpret_cast<uint4*>(xq_out + (int64_t)m * K + c * 16) =
                act_merge(*reinterpret_cast<const uint4*>(act + m * SLAB + act_chunk<NB>(c) * 16));
        }
    }
}

// FUSED: the activations arrive as bf16 rows x (rotated and quantised in the block, see
// rotate_quant_to_lds; K <= slab_cols(MM)) instead of xq / xs.
// CARRY: the tile's channel scales and biases are loaded with each batch (for blocks that
// walk several tiles); otherwise they are loaded once, in the tile's epilogue.
template <int MM, int R, int NB, bool FUSED = false, bool LONGK = false, bool CARRY = false, bool GROUPED = false>
__device__ __forceinline__ void gemv_body(const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                          const uint8_t* __restrict__ qp, const uint8_t* __restrict__ srel,
                                          const float* __restrict__ codebook, const float* __restrict__ ws,
                                          const float* __restrict__ bias, int N, int K, int out_type,
                                          void* __restrict__ out, int tile0, int ntile, int tstride,
                                          const uint16_t* __restrict__ x = nullptr, int qmax = 127,
                                          int8_t* __restrict__ xq_out = nullptr, float* __restrict__ xs_out = nullptr) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint32_t* lut = reinterpret_cast<uint32_t*>(smem);
    uint8_t* act = smem + 4096;
    const uint4* lut4 = reinterpret_cast<const uint4*>(lut);
    constexpr int SLAB = slab_cols(MM);
    constexpr int WAVES = GV_THREADS / 64;

    // the wave index as a uniform value, so row-dependent scalars use scalar loads
    // GROUPED (two instantiations of this body in one kernel): the thread index through an
    // opaque copy, so the compiler recomputes the lane-dependent addresses it derives where
    // they are used instead of keeping them all live (which spilled); the single-layer
    // kernels measured faster with the plain index
    int tid = (int)threadIdx.x;
    if constexpr (GROUPED) asm volatile("" : "+v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int KH = K >> 1, G = K >> 4, nchunk = K >> 4;
    // the work is a sequence of steps (tile t, batch gb): batch gb covers groups
    // 64*NB*gb .. 64*NB*(gb + 1) - 1 of each of the tile's rows; tile t covers rows
    // 4R*(tile0 + t*tstride) ..; wave w takes R consecutive rows of it
    static_assert(NB == 3 || NB == 4, "3 or 4 groups per lane");
    constexpr int BG = 64 * NB;   // groups per batch
    const int nbt = (nchunk + BG - 1) / BG;
    const int nsteps = ntile * nbt;
    // a step as (tile, batch), advanced by counting (no divisions; uniform, scalar)
    struct Pos {
        int t, gb;
    };
    auto advance = [&](Pos p) __attribute__((always_inline)) {
        return p.gb + 1 == nbt ? Pos{p.t + 1, 0} : Pos{p.t, p.gb + 1};
    };
    auto issue = [&](Batch<R, NB>& dst, Pos p) __attribute__((always_inline)) {
        if (p.t >= ntile) p = Pos{ntile - 1, nbt - 1};   // past the end: a harmless reload of the last step
        const int t = p.t, gb = p.gb;
        const uint8_t* qr[R];
        const uint8_t* sr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = min(((tile0 + t * tstride) * WAVES + wave) * R + r, N - 1);
            qr[r] = qp + (int64_t)n * KH;
            sr[r] = srel + (int64_t)n * G;
        }
        load_batch<R, NB>(dst, qr, sr, NB * lane + gb * BG, nchunk);
        if constexpr (CARRY) {
            // the epilogue operands travel with the batch: loaded at the tile's end, after
            // the next prefetch, the wait for them would drain that prefetch at every tile
            // boundary
            const float* bsrc = bias ? bias : ws;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int n = min(((tile0 + t * tstride) * WAVES + wave) * R + r, N - 1);
                dst.w[r] = ws[n];
                dst.b[r] = bsrc[n];
            }
        }
    };

    float* xs_w = reinterpret_cast<float*>(act + MM * SLAB);   // the rows' activation scales
    Batch<R, NB> bA, bB;
    if constexpr (FUSED) {
        // the first rotation inputs, then (after a compiler barrier that keeps this issue
        // order) the first weight batch: the rotation waits only for its own loads
        const RotIn first0 = rot_first_job<MM>(x, K, 0), first1 = rot_first_job<MM>(x, K, 1);
        __builtin_amdgcn_sched_barrier(0);
        issue(bA, Pos{0, 0});
        float cb[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) cb[c] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(codebook[c])));
        build_level_table_regs(lut, cb, tid, GV_THREADS);
        double* tbuf = reinterpret_cast<double*>(act + MM * SLAB + 32);
        rotate_quant_to_lds<MM, NB, LONGK>(act, xs_w, tbuf, reinterpret_cast<float*>(tbuf + ROTQ_TBUF_DOUBLES), x, K, qmax,
                                first0, first1, xq_out, xs_out);
    } else {
        // activation loads first, then the first weight batch: the wait before the
        // activation stores leaves the weight loads outstanding while the level table
        // is built from the codebook (uniform loads)
        const int cols0 = K < SLAB ? K : SLAB;
        const float xsv = xs[min(tid, MM - 1)];
        stage_acts<MM, NB>(act, xq, K, 0, cols0, tid, [&]() __attribute__((always_inline)) { issue(bA, Pos{0, 0}); });
        // scales in LDS: a lane-dependent index into a register array would put it in scratch memory
        if (tid < MM) xs_w[tid] = xsv;
        float cb[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) cb[c] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(codebook[c])));
        build_level_table_regs(lut, cb, tid, GV_THREADS);
    }
    __syncthreads();

    const float* xs_lds = xs_w;
    int32_t acc[R * MM];
    uint32_t id = 0x03020100u;   // identity byte selector, kept in a register
    asm volatile("" : "+v"(id));
    int slab_k0 = 0;

    // One step: prefetch the next step's batch into `nxt` (unconditionally, so the compiler
    // can count the loads in flight), multiply-accumulate `cur`, and finish the tile after
    // its last batch.  `live` is false only for the padding step of an odd count, which
    // only issues its (harmless) prefetch.
    auto body = [&](Pos pos, const Batch<R, NB>& cur, Batch<R, NB>& nxt, bool live, auto one_slab, auto prefetch)
                    __attribute__((always_inline)) {
        constexpr bool ONE = decltype(one_slab)::value;
        if (decltype(prefetch)::value) issue(nxt, advance(pos));
        if (!live) return;   // the padding step only keeps the load count even
        const int t = pos.t, gb = pos.gb;
        if (gb == 0) {
#pragma unroll
            for (int i = 0; i < R * MM; ++i) acc[i] = 0;
        }
        if (!ONE) {
            const int k0 = (gb * BG * 16 / SLAB) * SLAB;   // NB = 4 here: a batch never straddles slabs
            if (k0 != slab_k0) {                 // other slab of activations (uniform)
                slab_k0 = k0;
                const int cols = K - slab_k0 < SLAB ? K - slab_k0 : SLAB;
                __syncthreads();
                stage_acts<MM, NB>(act, xq, K, slab_k0, cols, tid, []() {});
                __syncthreads();
            }
        }
        const int jb = NB * lane + gb * BG;   // the lane's first group of the batch
        if (jb < nchunk) {                     // all NB groups, or none
            // NB = 4: chunks c0 + u (c0 = a multiple of 4) sit at act_chunk(c0) ^ u, one
            // address per batch and an xor per group; NB = 3: at c0 + u
            const int a0 = act_chunk<NB>(jb - (slab_k0 >> 4)) * 16;
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                uint4 a[MM];
                const int au = NB == 4 ? (a0 ^ (16 * u)) : a0 + 16 * u;
#pragma unroll
                for (int m = 0; m < MM; ++m) a[m] = *reinterpret_cast<const uint4*>(act + m * SLAB + au);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint4 tt = lut4[(cur.s[r] >> (8 * u)) & 0xFFu];
                    const uint2 d0 = decode_split(cur.q[r][2 * u], tt, id),
                                d1 = decode_split(cur.q[r][2 * u + 1], tt, id);
#pragma unroll
                    for (int m = 0; m < MM; ++m) {
                        int32_t sacc = acc[r * MM + m];
                        sacc = __builtin_amdgcn_sdot4((int)d0.x, (int)a[m].x, sacc, false);
                        sacc = __builtin_amdgcn_sdot4((int)d0.y, (int)a[m].y, sacc, false);
                        sacc = __builtin_amdgcn_sdot4((int)d1.x, (int)a[m].z, sacc, false);
                        sacc = __builtin_amdgcn_sdot4((int)d1.y, (int)a[m].w, sacc, false);
                        acc[r * MM + m] = sacc;
                    }
                }
            }
        }
        if (gb == nbt - 1) {
            // reduce-scatter of the V = R*MM partial sums over the 64 lanes: after the
            // halving steps lane l holds value l >> (6 - L) summed over its 2^(6-L) group
            constexpr int V = R * MM, VP = pow2_ceil(V), L = log2i(VP);
            static_assert(VP <= 64, "too many partial sums per wave");
            int32_t v[VP];
#pragma unroll
            for (int i = 0; i < VP; ++i) v[i] = i < V ? acc[i] : 0;
#pragma unroll
            for (int st = 0; st < L; ++st) {
                const int o = 32 >> st, half = VP >> (st + 1);
                // lanes with bit o set keep the upper half; the swap is masked xor
                // arithmetic on an opaque mask (a select here is folded into a
                // lane-dependent index into v, i.e. a compare chain over all of it)
                int32_t hm = -((lane >> (5 - st)) & 1);
                asm volatile("" : "+v"(hm));
#pragma unroll
                for (int i = 0; i < half; ++i) {
                    const int32_t d = (v[i] ^ v[i + half]) & hm;
                    const int32_t keep = v[i] ^ d, send = v[i + half] ^ d;
                    v[i] = keep + lane_xor(send, o, lane);
                }
            }
            // then the sum over the 64 >> L lanes that share a value: within a 16-lane row by
            // DPP (quad xor 1 and xor 2, then the half-row mirror pairs quads, the row mirror
            // pairs half-rows), across rows by lane shuffles; every lane ends with the sum
            constexpr int G = 64 >> L;
            if constexpr (G >= 2) v[0] += __builtin_amdgcn_update_dpp(0, v[0], 0xB1, 0xF, 0xF, false);
            if constexpr (G >= 4) v[0] += __builtin_amdgcn_update_dpp(0, v[0], 0x4E, 0xF, 0xF, false);
            if constexpr (G >= 8) v[0] += __builtin_amdgcn_update_dpp(0, v[0], 0x141, 0xF, 0xF, false);
            if constexpr (G >= 16) v[0] += __builtin_amdgcn_update_dpp(0, v[0], 0x140, 0xF, 0xF, false);
            if constexpr (G >= 32) v[0] += lane_xor(v[0], 16, lane);
            if constexpr (G >= 64) v[0] += lane_xor(v[0], 32, lane);

            const int n0 = ((tile0 + t * tstride) * WAVES + wave) * R;
            const int idx = lane >> (6 - L);
            const int r = idx / MM, m = idx - r * MM;
            float wv[R], bv[R];
#pragma unroll
            for (int i = 0; i < R; ++i) {
                if constexpr (CARRY) {
                    wv[i] = cur.w[i];
                    bv[i] = cur.b[i];
                } else {   // wave-uniform addresses
                    wv[i] = ws[min(n0 + i, N - 1)];
                    bv[i] = bias ? bias[min(n0 + i, N - 1)] : 0.0f;
                }
            }
            float wn = wv[0], bn = bv[0];
#pragma unroll
            for (int i = 1; i < R; ++i) {
                wn = r == i ? wv[i] : wn;
                bn = r == i ? bv[i] : bn;
            }
            const float xm = xs_lds[m < MM ? m : 0];
            const int n = n0 + r;
            const bool lead = (lane & ((1 << (6 - L)) - 1)) == 0 && idx < V && n < N;
            float y = __fmul_rn((float)v[0], __fmul_rn(xm, wn));
            if (bias) y = __fadd_rn(y, bn);
            if (out_type == 3) {
                // SwiGLU (two rows per wave): the gate row n0 (r = 0) takes the up row n0 + 1
                // from the lane holding (r = 1, m), MM values further on
                const float u = __shfl(y, lane + (MM << (6 - L)), 64);
                if (lead && r == 0)
                    reinterpret_cast<uint16_t*>(out)[(int64_t)m * (N >> 1) + (n >> 1)] = f32_to_bf16(swiglu_f32(y, u));
            } else if (lead) {
                store_out(out, out_type, (int64_t)m * N + n, v[0], y);
            }
        }
    };
    auto run = [&](auto one_slab) __attribute__((always_inline)) {
        Pos pos{0, 0};
        for (int step = 0; step < nsteps; step += 2) {   // ping-pong: no register copies
            body(pos, bA, bB, true, one_slab, std::true_type{});
            pos = advance(pos);
            body(pos, bB, bA, step + 1 < nsteps, one_slab, std::true_type{});
            pos = advance(pos);
        }
    };
    if (nsteps == 1) body(Pos{0, 0}, bA, bB, true, std::true_type{}, std::false_type{});   // one tile, one batch
    else if (FUSED || K <= SLAB) run(std::true_type{});
    else if constexpr (!FUSED && NB == 4) run(std::false_type{});   // 3 groups per lane: one slab only
}

// for one activation row, at most 128 registers (4 waves per SIMD; 131 registers, 3 waves,
// measured 0.9 us slower at N = K = 4096)
template <int MM, int R, int NB>
__global__ __launch_bounds__(GV_THREADS, MM == 1 ? 4 : 1) void gemv_kernel(const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                                          const uint8_t* __restrict__ qp,
                                                          const uint8_t* __restrict__ srel,
                                                          const float* __restrict__ codebook,
                                                          const float* __restrict__ ws,
                                                          const float* __restrict__ bias, int N, int K,
                                                          int out_type, void* __restrict__ out) {
    // carrying the epilogue operands measured faster for several rows, slower for one
    gemv_body<MM, R, NB, false, false, (MM > 1)>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, blockIdx.x,
                                                 1, 1);
}

template <int MM, int R, int NB, bool LONGK>
__global__ __launch_bounds__(GV_THREADS) void gemv_act_kernel(const uint16_t* __restrict__ x, int qmax,
                                                              const uint8_t* __restrict__ qp,
                                                              const uint8_t* __restrict__ srel,
                                                              const float* __restrict__ codebook,
                                                              const float* __restrict__ ws,
                                                              const float* __restrict__ bias, int N, int K,
                                                              int out_type, void* __restrict__ out,
                                                              int8_t* __restrict__ xq_out, float* __restrict__ xs_out) {
    const bool first = blockIdx.x == 0;   // one block writes the prepared activations out
    gemv_body<MM, R, NB, true, LONGK>(nullptr, nullptr, qp, srel, codebook, ws, bias, N, K, out_type, out, blockIdx.x, 1,
                                      1, x, qmax, first ? xq_out : nullptr, first ? xs_out : nullptr);
}

// Several independent layers (same M) in one launch: block b works on the layer whose
// range [first[l], first[l+1]) of block ids holds b, as block b - first[l] of it, on
// every nblk-th row tile of the layer (the level table and the activations are staged
// once per block; the first loads of a tile are issued during the last batch of the
// previous one).  The blocks running at one time thus read neighbouring rows of one
// layer.  The layer table travels in the kernel arguments (about 5.5 KB), with each
// layer's groups per lane and batch (gemv_nb).
struct GroupArgs {
    int count;
    int first[GEMV_GROUP_MAX + 1];
    uint8_t nb[GEMV_GROUP_MAX];
    w4a8_gemv_layer layer[GEMV_GROUP_MAX];
};

// for one activation row, at most 128 registers (4 waves per SIMD, measured faster than 3)
template <int MM, int R>
__global__ __launch_bounds__(GV_THREADS, MM == 1 ? 4 : 1) void gemv_grouped_kernel(const GroupArgs args, int out_type) {
    // the layer: the last l with first[l] <= block id (binary search, uniform)
    int l = 0;
    for (int hi = args.count - 1; l < hi;) {
        const int mid = (l + hi + 1) >> 1;
        if (args.first[mid] <= (int)blockIdx.x) l = mid;
        else hi = mid - 1;
    }
    const w4a8_gemv_layer& L = args.layer[l];
    const int per_tile = (GV_THREADS / 64) * R;
    const int tiles = (int)((L.N + per_tile - 1) / per_tile);
    const int nblk = args.first[l + 1] - args.first[l], bl = (int)blockIdx.x - args.first[l];
    const int ntile = (tiles - bl + nblk - 1) / nblk;
    if (args.nb[l] == 3)   // block-uniform
        gemv_body<MM, R, 3, false, false, true, true>(L.xq, L.xs, L.qpacked, L.srel, L.codebook, L.s_channel, L.bias,
                                                (int)L.N, (int)L.K, out_type, L.out, bl, ntile, nblk);
    else
        gemv_body<MM, R, 4, false, false, true, true>(L.xq, L.xs, L.qpacked, L.srel, L.codebook, L.s_channel, L.bias,
                                                (int)L.N, (int)L.K, out_type, L.out, bl, ntile, nblk);
}

// rows per wave: 2 when that still gives >= 2048 waves (8 per compute unit), else 1
// (4 rows per wave would need so many registers that few waves fit per SIMD)
int rows_per_wave(int64_t rows) { return (rows + 1) / 2 >= 2048 ? 2 : 1; }

// Blocks of gemv_grouped_kernel<MM, R> that are resident on one compute unit at a time
// (from the runtime's occupancy calculation; cached, the same for every gfx950 device).
template <int MM, int R>
int grouped_blocks_per_cu() {
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemv_grouped_kernel<MM, R>, GV_THREADS,
                                                         gemv_lds_bytes(MM, false)) != hipSuccess || n < 1)
            n = 1;
        cached.store(n, std::memory_order_relaxed);
        v = n;
    }
    return v;
}

template <int MM>
hipError_t launch_gemv_grouped_m(const w4a8_gemv_layer* layers, int count, int out_type, hipStream_t stream) {
    int64_t rows = 0;
    for (int i = 0; i < count; ++i) rows += layers[i].N;
    const int R = out_type == 3 ? 2 : rows_per_wave(rows), per_tile = (GV_THREADS / 64) * R;   // SwiGLU pairs rows
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t slots = (int64_t)cus * (R == 2 ? grouped_blocks_per_cu<MM, 2>() : grouped_blocks_per_cu<MM, 1>());
    // A tile of layer i costs cost(i) (its weight batches of 3 or 4 groups per lane, plus about
    // one for the epilogue).  Each launch is cut into at most GV_ROUNDS rounds of `slots`
    // blocks of about equal cost: the blocks of a layer take its tiles round robin, and the
    // block counts are rounded down, so no block starts in a partial last round.
    auto nb_of = [&](const w4a8_gemv_layer& L) { return gemv_nb((int)L.K, slab_cols(MM)); };
    auto tiles_of = [&](const w4a8_gemv_layer& L) { return (L.N + per_tile - 1) / per_tile; };
    auto cost_of = [&](const w4a8_gemv_layer& L) {
        const int nb = nb_of(L);
        return (L.K / 16 + 64 * nb - 1) / (64 * nb) * nb + 1;
    };
    for (int base = 0; base < count; base += GEMV_GROUP_MAX) {
        GroupArgs a;
        a.count = count - base < GEMV_GROUP_MAX ? count - base : GEMV_GROUP_MAX;
        int64_t total = 0;
        for (int i = 0; i < a.count; ++i) total += tiles_of(layers[base + i]) * cost_of(layers[base + i]);
        const int64_t target = GV_ROUNDS * slots;
        a.first[0] = 0;
        for (int i = 0; i < a.count; ++i) {
            const w4a8_gemv_layer& L = layers[base + i];
            a.layer[i] = L;
            a.nb[i] = (uint8_t)nb_of(L);
            const int64_t t = tiles_of(L);
            int64_t n = t * cost_of(L) * target / total;
            n = n < 1 ? 1 : n > t ? t : n;
            a.first[i + 1] = a.first[i] + (int)n;
        }
        for (int i = a.count; i < GEMV_GROUP_MAX; ++i) {
            a.first[i + 1] = a.first[a.count];
            a.nb[i] = 4;
        }
        const size_t lds = gemv_lds_bytes(MM, false);
        const dim3 g(a.first[a.count]), b(GV_THREADS);
        if (R == 2)
            hipLaunchKernelGGL((gemv_grouped_kernel<MM, 2>), g, b, lds, stream, a, out_type);
        else
            hipLaunchKernelGGL((gemv_grouped_kernel<MM, 1>), g, b, lds, stream, a, out_type);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int MM>
hipError_t launch_gemv_m(const int8_t* xq, const float* xs, const uint8_t* qp, const uint8_t* srel,
                         const float* codebook, const float* ws, const float* bias, int N, int K, int out_type,
                         void* out, hipStream_t stream) {
    const int waves_per_block = GV_THREADS / 64;
    const int R = out_type == 3 ? 2 : rows_per_wave(N);   // SwiGLU pairs the rows of a wave
    const int blocks = (N + waves_per_block * R - 1) / (waves_per_block * R);
    const size_t lds = gemv_lds_bytes(MM, false);
    const dim3 g(blocks), b(GV_THREADS);
    const int nb = gemv_nb(K, slab_cols(MM));
#define GV_LAUNCH(RR, NBV)                                                                                           \
    hipLaunchKernelGGL((gemv_kernel<MM, RR, NBV>), g, b, lds, stream, xq, xs, qp, srel, codebook, ws, bias, N, K, \
                       out_type, out)
    if (R == 2) {
        if (nb == 3) GV_LAUNCH(2, 3); else GV_LAUNCH(2, 4);
    } else {
        if (nb == 3) GV_LAUNCH(1, 3); else GV_LAUNCH(1, 4);
    }
#undef GV_LAUNCH
    return hipGetLastError();
}

template <int MM>
hipError_t launch_gemv_act_m(const uint16_t* x, int qmax, const uint8_t* qp, const uint8_t* srel,
                             const float* codebook, const float* ws, const float* bias, int N, int K, int out_type,
                             void* out, int8_t* xq_out, float* xs_out, hipStream_t stream) {
    const int waves_per_block = GV_THREADS / 64;
    const int R = out_type == 3 ? 2 : rows_per_wave(N);   // SwiGLU pairs the rows of a wave
    const int blocks = (N + waves_per_block * R - 1) / (waves_per_block * R);
    const size_t lds = gemv_lds_bytes(MM, true);
    const dim3 g(blocks), b(GV_THREADS);
    const int nb = gemv_nb(K, slab_cols(MM));
#define GV_ACT_LAUNCH(RR, NBV, LL)                                                                               \
    hipLaunchKernelGGL((gemv_act_kernel<MM, RR, NBV, LL>), g, b, lds, stream, x, qmax, qp, srel, codebook, ws, bias, \
                       N, K, out_type, out, xq_out, xs_out)
#define GV_ACT_NB(RR, LL)                  \
    if (nb == 3) GV_ACT_LAUNCH(RR, 3, LL); \
    else GV_ACT_LAUNCH(RR, 4, LL)
    if constexpr (slab_cols(MM) > 4096) {
        if (K > 4096) {
            if (R == 2) { GV_ACT_NB(2, true); }
            else { GV_ACT_NB(1, true); }
            return hipGetLastError();
        }
    }
    if (R == 2) { GV_ACT_NB(2, false); }
    else { GV_ACT_NB(1, false); }
#undef GV_ACT_NB
#undef GV_ACT_LAUNCH
    return hipGetLastError();
}

}  // namespace

int gemv_act_max_k(int M) { return M >= 1 && M <= 8 ? slab_cols(M) : 0; }

hipError_t launch_gemv_act(const uint16_t* x, int M, int qmax, const uint8_t* qp, const uint8_t* srel,
                           const float* codebook, const float* ws, const float* bias, int N, int K, int out_type,
                           void* out, int8_t* xq_out, float* xs_out, hipStream_t stream) {
    (void)hipGetLastError();   // clear a stale error so the check below is about this launch
    switch (M) {
#define GV_ACT_CASE(MMV) \
        case MMV: return launch_gemv_act_m<MMV>(x, qmax, qp, srel, codebook, ws, bias, N, K, out_type, out, xq_out, xs_out, stream);
        GV_ACT_CASE(1) GV_ACT_CASE(2) GV_ACT_CASE(3) GV_ACT_CASE(4)
        GV_ACT_CASE(5) GV_ACT_CASE(6) GV_ACT_CASE(7) GV_ACT_CASE(8)
#undef GV_ACT_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_grouped(const w4a8_gemv_layer* layers, int count, int M, int out_type, hipStream_t stream) {
    (void)hipGetLastError();   // clear a stale error so the checks below are about these launches
    switch (M) {
        case 1: return launch_gemv_grouped_m<1>(layers, count, out_type, stream);
        case 2: return launch_gemv_grouped_m<2>(layers, count, out_type, stream);
        case 3: return launch_gemv_grouped_m<3>(layers, count, out_type, stream);
        case 4: return launch_gemv_grouped_m<4>(layers, count, out_type, stream);
        case 5: return launch_gemv_grouped_m<5>(layers, count, out_type, stream);
        case 6: return launch_gemv_grouped_m<6>(layers, count, out_type, stream);
        case 7: return launch_gemv_grouped_m<7>(layers, count, out_type, stream);
        case 8: return launch_gemv_grouped_m<8>(layers, count, out_type, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(const int8_t* xq, const float* xs, int M, const uint8_t* qp, const uint8_t* srel,
                       const float* codebook, const float* ws, const float* bias, int N, int K, int out_type,
                       void* out, hipStream_t stream) {
    (void)hipGetLastError();   // clear a stale error so the check below is about this launch
    switch (M) {
        case 1: return launch_gemv_m<1>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 2: return launch_gemv_m<2>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 3: return launch_gemv_m<3>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 4: return launch_gemv_m<4>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 5: return launch_gemv_m<5>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 6: return launch_gemv_m<6>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 7: return launch_gemv_m<7>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        case 8: return launch_gemv_m<8>(xq, xs, qp, srel, codebook, ws, bias, N, K, out_type, out, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a8
