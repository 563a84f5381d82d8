// gfx950 kernels of the PCD hot path.
//
// Matrix work runs on the CDNA4 matrix cores: v_mfma_f32_16x16x32_bf16 for
// bf16 models and v_mfma_f32_16x16x4_f32 for fp32 models, always with fp32
// accumulation.  A lane of a 64-wide wavefront owns 8 consecutive k-elements
// of one A row and of one B column (lane%16 picks the row/column, lane/16 the
// k-octet); which k-octet goes to which lane group only has to agree between A
// and B, so both operands use the same map.  The 16x16 accumulator of a lane
// holds rows 4*(lane/16)+i, i<4, of column lane%16.
#include "pcd_kernels.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>
#include <utility>

namespace pcd {

typedef uint16_t bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int PCD_DT_F32 = 0;

// ---------------------------------------------------------------------------
// element conversion (bf16 is stored as its 16-bit pattern)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
// round to nearest, ties to even: one v_cvt_pk_bf16_f32 on gfx950 (two values
// per instruction where the compiler can pair them)
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return __builtin_bit_cast(bf16_t, (__bf16)v); }

// 8 consecutive elements of one MFMA operand row/column
template <typename T> struct Frag;
template <> struct Frag<bf16_t> { bf16x8_t v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void ld8(Frag<bf16_t> &f, const bf16_t *p) { f.v = *reinterpret_cast<const bf16x8_t *>(p); }
__device__ __forceinline__ void ld8(Frag<float> &f, const float *p) {
    const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
// two runs of 4 elements (used for the P*V operand)
__device__ __forceinline__ void ld4x2(Frag<bf16_t> &f, const bf16_t *p0, const bf16_t *p1) {
    const uint2 a = *reinterpret_cast<const uint2 *>(p0), b = *reinterpret_cast<const uint2 *>(p1);
    u32x4 u = {a.x, a.y, b.x, b.y};
    f.v = __builtin_bit_cast(bf16x8_t, u);
}
__device__ __forceinline__ void ld4x2(Frag<float> &f, const float *p0, const float *p1) {
    const float4 a = *reinterpret_cast<const float4 *>(p0), b = *reinterpret_cast<const float4 *>(p1);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
// 8 floats to bf16 (round to nearest even), two per packed conversion
typedef float float2v_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void from8(Frag<bf16_t> &f, const float *x) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float2v_t v = {x[2 * i], x[2 * i + 1]};
        u[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
    }
    f.v = __builtin_bit_cast(bf16x8_t, u);
}
__device__ __forceinline__ void from8(Frag<float> &f, const float *x) {
    for (int i = 0; i < 8; ++i) f.v[i] = x[i];
}

// 8 floats to 8 consecutive elements at p (16-byte aligned), in 16-byte stores
__device__ __forceinline__ void store8(bf16_t *p, const float *x) {
    Frag<bf16_t> f;
    from8(f, x);
    *reinterpret_cast<bf16x8_t *>(p) = f.v;
}
__device__ __forceinline__ void store8(float *p, const float *x) {
    reinterpret_cast<float4 *>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

__device__ __forceinline__ void mma(f32x4 &acc, const Frag<bf16_t> &a, const Frag<bf16_t> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4 &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Reductions across the four 16-lane rows of a wave with gfx950's row swaps
// (no LDS round trip): v_permlane16_swap pairs rows (0,1) and (2,3),
// v_permlane32_swap pairs the two halves; combining a value with its swapped
// copies leaves the result for its 16-lane column in every row.
__device__ __forceinline__ float rows_max(float v) {
    const uint32_t u = __float_as_uint(v);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t w = __float_as_uint(v);
    auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
    const uint32_t u = __float_as_uint(v);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t w = __float_as_uint(v);
    auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// GEMM  C[M][N] = A[M][K] . B[N][K]^T  with a fused epilogue
//
// Both operands stream through an S-stage ring of LDS tiles, filled straight
// from global memory by gfx950's global_load_lds_dwordx4 (each lane's 16
// bytes land at M0 + 16*lane), so S-1 k-tiles are in flight while the
// matrix cores work on the current one and no registers stage the copies.
// A tile row holds 128 bytes of K (8 chunks of 16 B); chunk c of row r is
// stored in slot c ^ (r % 8) of that row, which makes the 16-byte fragment
// reads of 8 consecutive rows hit 8 disjoint bank groups.  One barrier per
// k-tile: after it, every wave has finished the previous tile, whose slot is
// then refilled.
// ---------------------------------------------------------------------------
template <int NB> struct GemmArgs {
    const void *A;
    BSegs B[NB];
    int32_t M, N, K;
    int32_t tiles_m, tiles_n, splits, k_per_split, total, per_xcd;
    int32_t stagger;  // k-stages by which each row tile's k order is rotated against the previous one
    int32_t b_once;   // one row tile: every B line is read once (non-temporal loads)
};

struct EpiArgs {
    float *x, *part;
    void *out, *kc, *vc, *kc2, *vc2;
    int32_t cap, cap2, kv_split, n_q, n_k, hd;
    const int32_t *kv_req, *kv_row, *kv_cap;
    const uint64_t *kv_base;
    int32_t kv_layer;
    const int32_t *pos;
    const float2 *rope;
    float2 *ro_part;
    const int32_t *g_tok, *g_ro;
    int32_t n_gather;
    float *g_logit;
};

__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// 16 bytes per lane from global memory into LDS at lds_addr + 16 * lane.
// Issued from inline assembly so that the compiler does not add a wait for
// it before every LDS read; completion is tracked by vm_wait below.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds_addr) {
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_addr) : "memory");
}
// The same with the non-temporal hint: for data read once, which then
// leaves L2 first instead of pushing out lines that will be read again.
__device__ __forceinline__ void dma16_nt(const void *g, uint32_t lds_addr) {
    asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(lds_addr) : "memory");
}
// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int... Is, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, F &&f) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F> __device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(std::make_integer_sequence<int, N>{}, f);
}
// wait until at most N vector-memory operations of this wave are in flight
template <int N> __device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// vm_wait<ahead * LPS> for a run-time ahead in [0, A]
template <int LPS, int A> __device__ __forceinline__ void vm_wait_ahead(int ahead) {
    if constexpr (A <= 0) {
        vm_wait<0>();
    } else {
        if (ahead >= A) vm_wait<A * LPS>();
        else vm_wait_ahead<LPS, A - 1>(ahead);
    }
}
// wait until this wave's LDS reads have returned (lgkmcnt 0; vmcnt untouched)
__device__ __forceinline__ void lds_reads_done() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// workgroup barrier that does not wait for in-flight global loads
__device__ __forceinline__ void barrier_keep_loads() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <typename T, int BM, int BN, int NB, Epi E, int KB = 128> struct GemmLds {
    static constexpr bool LDS_EPI = (E == Epi::Qkv || E == Epi::Readout);
    static constexpr int STAGE = (BM + NB * BN) * KB;
    // Qkv: after the C tile, per row its position and the destinations of up
    // to 4 heads (BN = 128 columns of heads of at least 32)
    static constexpr int META = E == Epi::Qkv ? BM * (4 + 4 * 8) : 0;
    static constexpr int C_BYTES = LDS_EPI ? BM * (BN + 4) * 4 + META : 0;
    static int bytes(int S) { return S * STAGE > C_BYTES ? S * STAGE : C_BYTES; }
};

template <typename T, int BM, int BN, int WM, int WN, int NB, int S, Epi E, int KB = 128, bool ILV = false>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm(GemmArgs<NB> g, EpiArgs e) {
    constexpr int NW = WM * WN;         // waves per workgroup
    constexpr int NT = NW * 64;
    constexpr int CH = 16 / sizeof(T);  // elements per 16-byte chunk
    constexpr int CPR = KB / 16;        // chunks per tile row per stage
    constexpr int BK = CPR * CH;        // K elements per stage
    constexpr int A_BYTES = BM * KB, B_BYTES = BN * KB, STAGE = A_BYTES + NB * B_BYTES;
    // DMA instructions per wave per stage.  A tile whose rows do not split
    // evenly over the waves (BM a multiple of 8, not of 8 NW) leaves the last
    // instruction to the first A_GRP % NW waves only; the waits count the
    // smaller number, which can only make a wave wait longer than it must.
    constexpr int A_GRP = BM * CPR / 64;  // 64-lane groups of 16-byte chunks in one A stage
    constexpr int A_INS = (A_GRP + NW - 1) / NW, B_INS = BN * CPR / (64 * NW);
    constexpr int LPS = A_GRP / NW + NB * B_INS;
    constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 16, FN = WTN / 16;
    constexpr int KSTEPS = BK / 32;
    constexpr int CPL = 8 / CH;  // chunks holding one lane's 8 k-elements
    constexpr bool LDS_EPI = GemmLds<T, BM, BN, NB, E, KB>::LDS_EPI;
    static_assert((NW == 4 || NW == 8) && (KB == 128 || KB == 256), "workgroup shape");
    static_assert(A_GRP * 64 == BM * CPR && B_INS * 64 * NW == BN * CPR, "tile rows per DMA instruction");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
    static_assert(S >= 2 && S <= 8 && (S - 1) * (A_INS + NB * B_INS) < 64, "pipeline depth");
    static_assert(S * STAGE <= 160 * 1024, "operand ring exceeds the 160 KB of LDS");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds;

    // XCD-aware tile order: consecutive workgroups land on different XCDs, so
    // hand each XCD a contiguous range of tiles (m fastest): tiles that share
    // a B slab run on one XCD and share its L2.
    const int b = blockIdx.x;
    const int t = (b & 7) * g.per_xcd + (b >> 3);
    if (t >= g.total) return;
    const int tm = t % g.tiles_m;
    const int rest = t / g.tiles_m;
    const int ks = rest % g.splits;
    const int tn = rest / g.splits;
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = ks * g.k_per_split;
    const int nkt = g.k_per_split / BK;

    // the wave index is uniform: LDS addresses of the DMAs stay in scalar registers
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w % WM, wn = w / WM;
    const int lr = lane & 15, lg = lane >> 4;

    // DMA sources: slot p = (i*NW + w)*64 + lane of a tile is row p/CPR, chunk (p%CPR) ^ (row%8)
    const T *A = reinterpret_cast<const T *>(g.A);
    const char *asrc[A_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        const int p = (i * NW + w) * 64 + lane, r = p / CPR, c = (p % CPR) ^ (r & 7);
        const int m = min(m0 + r, g.M - 1);  // rows past M load row M-1; their results are dropped
        asrc[i] = reinterpret_cast<const char *>(A + (size_t)m * g.K + kbeg + c * CH);
    }
    const char *bsrc[NB][B_INS];
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int i = 0; i < B_INS; ++i) {
            const int p = (i * NW + w) * 64 + lane, r = p / CPR, c = (p % CPR) ^ (r & 7);
            const int n = min(n0 + r, g.N - 1);  // rows past N (a ragged last readout tile) load row N-1, unused
            const BSegs &sg = g.B[q];
            const int s = (sg.nseg > 2 && n >= sg.begin[2]) ? 2 : ((sg.nseg > 1 && n >= sg.begin[1]) ? 1 : 0);
            bsrc[q][i] = reinterpret_cast<const char *>(reinterpret_cast<const T *>(sg.ptr[s]) +
                                                         (size_t)(n - sg.begin[s]) * g.K + kbeg + c * CH);
        }
    // The row tiles of one column slab run at once on one XCD and read the
    // same weight lines; each starts its k loop `stagger` stages after the
    // previous row tile's start (in a rotated order), so that most of them
    // read lines another one fetched a few stages earlier, from L2.
    const int rot = nkt > 0 ? (int)(((int64_t)tm * g.stagger) % nkt) : 0;
    auto issue = [&](int kt) {
        const uint32_t sb = lds_base + (uint32_t)((kt % S) * STAGE);
        const int kk = kt + rot;
        const size_t ko = (size_t)(kk >= nkt ? kk - nkt : kk) * KB;
#pragma unroll
        for (int i = 0; i < A_INS; ++i)
            if (A_GRP % NW == 0 || i * NW + w < A_GRP) dma16(asrc[i] + ko, sb + (uint32_t)((i * NW + w) * 1024));
        auto issue_b = [&](auto NT) {
#pragma unroll
            for (int q = 0; q < NB; ++q)
#pragma unroll
                for (int i = 0; i < B_INS; ++i) {
                    const uint32_t dst = sb + (uint32_t)(A_BYTES + q * B_BYTES + (i * NW + w) * 1024);
                    if constexpr (decltype(NT)::value) dma16_nt(bsrc[q][i] + ko, dst);
                    else dma16(bsrc[q][i] + ko, dst);
                }
        };
        // the readout of a few rows (one row tile) streams the LM head once
        if constexpr (E == Epi::Readout && BM <= 64) {
            if (g.b_once) issue_b(std::true_type{});
            else issue_b(std::false_type{});
        } else {
            issue_b(std::false_type{});
        }
    };
    // DMA instruction d of stage kt alone: A rows first, then each B operand's rows
    constexpr int LPI = A_INS + NB * B_INS;  // this wave's DMA instructions per stage, at most
    auto issue_one = [&](int kt, auto D) {
        constexpr int d = decltype(D)::value;
        const uint32_t sb = lds_base + (uint32_t)((kt % S) * STAGE);
        const int kk = kt + rot;
        const size_t ko = (size_t)(kk >= nkt ? kk - nkt : kk) * KB;
        if constexpr (d < A_INS) {
            if (A_GRP % NW == 0 || d * NW + w < A_GRP) dma16(asrc[d] + ko, sb + (uint32_t)((d * NW + w) * 1024));
        } else {
            constexpr int q = (d - A_INS) / B_INS, i = (d - A_INS) % B_INS;
            const uint32_t dst = sb + (uint32_t)(A_BYTES + q * B_BYTES + (i * NW + w) * 1024);
            if constexpr (E == Epi::Readout && BM <= 64) {
                if (g.b_once) dma16_nt(bsrc[q][i] + ko, dst);
                else dma16(bsrc[q][i] + ko, dst);
            } else {
                dma16(bsrc[q][i] + ko, dst);
            }
        }
    };
    auto frag = [&](Frag<T> &f, const char *tile, int row, int chunk) {
        const char *p0 = tile + (row * CPR + (chunk ^ (row & 7))) * 16;
        if constexpr (CPL == 1) {
            ld8(f, reinterpret_cast<const T *>(p0));
        } else {
            const char *p1 = tile + (row * CPR + ((chunk + 1) ^ (row & 7))) * 16;
            ld4x2(f, reinterpret_cast<const T *>(p0), reinterpret_cast<const T *>(p1));
        }
    };

    f32x4 acc[NB][FM][FN];
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[q][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Fragments are double-buffered in registers: the LDS reads of the next
    // k-step go out before the matrix-core work of the current one, and the
    // per-tile wait + barrier sit between two MFMA batches.  Stage kt lives in
    // slot kt % S; S stages are issued ahead; stage kt+S refills slot kt % S
    // right after the barrier that follows the last read of stage kt.
    Frag<T> fa[2][FM], fb[2][NB][FN];
    auto read_frags = [&](auto BUF, int kt, int s) {
        constexpr int bb = decltype(BUF)::value;
        const char *st = lds + (kt % S) * STAGE;
#pragma unroll
        for (int i = 0; i < FM; ++i) frag(fa[bb][i], st, wm * WTM + i * 16 + lr, s * 4 * CPL + lg * CPL);
#pragma unroll
        for (int q = 0; q < NB; ++q)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                frag(fb[bb][q][j], st + A_BYTES + q * B_BYTES, wn * WTN + j * 16 + lr, s * 4 * CPL + lg * CPL);
    };
    // matrix instructions [lo, hi) of one k-step, in (q, j, i) order
    constexpr int NM = NB * FN * FM;
    auto mfmas = [&](auto BUF, auto LO, auto HI) {
        constexpr int bb = decltype(BUF)::value, lo = decltype(LO)::value, hi = decltype(HI)::value;
#pragma unroll
        for (int q = 0; q < NB; ++q)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int idx = (q * FN + j) * FM + i;
                    if (idx >= lo && idx < hi) mma(acc[q][i][j], fa[bb][i], fb[bb][q][j]);
                }
    };
    static_assert(KSTEPS % 2 == 0, "k-steps per stage must be even for the fragment ping-pong");
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using M0 = std::integral_constant<int, 0>;
    using MH = std::integral_constant<int, NM / 4>;
    using MN = std::integral_constant<int, NM>;

    // One stage, k-steps in pairs: buffer 0 computes while buffer 1 loads and
    // the reverse.  The order within a pair is pinned (sched_barrier): a
    // quarter of buffer 0's matrix instructions, the LDS reads of buffer 1,
    // the rest of buffer 0, then (after the stage's last k-step) the refill
    // of the slot just consumed, the reads of the next stage's first k-step,
    // and buffer 1's matrix instructions.  So no wait ever covers reads issued
    // for a later k-step, and each read has a run of matrix instructions to
    // land behind.  KIND 0: S-2 later stages in flight, refill stage kt+S;
    // KIND 1 (the last stages): wait for everything, no refill; KIND 2: the
    // final stage, nothing follows.
    auto stage = [&](int kt, auto KIND) {
        constexpr int kind = decltype(KIND)::value;
#pragma unroll
        for (int s = 0; s < KSTEPS; s += 2) {
            mfmas(B0{}, M0{}, MH{});
            __builtin_amdgcn_sched_barrier(0);
            read_frags(B1{}, kt, s + 1);
            __builtin_amdgcn_sched_barrier(0);
            mfmas(B0{}, MH{}, MN{});
            if (s + 2 < KSTEPS) {
                read_frags(B0{}, kt, s + 2);
            } else if constexpr (kind != 2) {
                __builtin_amdgcn_sched_barrier(0);
                // this wave's reads of stage kt must be done before anyone refills its slot
                lds_reads_done();
                if constexpr (kind == 0) vm_wait<(S - 2) * LPS>();
                else vm_wait<0>();
                barrier_keep_loads();
                if constexpr (kind == 0 && !ILV) issue(kt + S);
                read_frags(B0{}, kt + 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (ILV && kind == 0) {
                if (s + 2 >= KSTEPS) {
                    // the refill's DMA instructions one at a time between runs of
                    // buffer 1's matrix instructions, not in one burst ahead of them
                    static_for<LPI>([&](auto D) {
                        constexpr int d = decltype(D)::value;
                        mfmas(B1{}, std::integral_constant<int, d * NM / LPI>{},
                              std::integral_constant<int, (d + 1) * NM / LPI>{});
                        __builtin_amdgcn_sched_barrier(0);
                        issue_one(kt + S, D);
                        __builtin_amdgcn_sched_barrier(0);
                    });
                } else {
                    mfmas(B1{}, M0{}, MN{});
                }
            } else {
                mfmas(B1{}, M0{}, MN{});
            }
        }
    };

#pragma unroll
    for (int s = 0; s < S; ++s)
        if (s < nkt) issue(s);
    // stage 0 landed; the S-1 stages issued after it may stay in flight
    if (nkt >= S) vm_wait<(S - 1) * LPS>();
    else vm_wait<0>();
    barrier_keep_loads();
    read_frags(B0{}, 0, 0);
    int kt = 0;
    for (; kt + S < nkt; ++kt) stage(kt, std::integral_constant<int, 0>{});
    for (; kt + 1 < nkt; ++kt) stage(kt, std::integral_constant<int, 1>{});
    stage(kt, std::integral_constant<int, 2>{});

    if constexpr (!LDS_EPI) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + wm * WTM + i * 16 + lg * 4 + r;
                    const int n = n0 + wn * WTN + j * 16 + lr;
                    if (m >= g.M) continue;
                    if constexpr (E == Epi::Resid) {
                        e.x[(size_t)m * g.N + n] += acc[0][i][j][r];
                    } else if constexpr (E == Epi::Partial) {
                        e.part[((size_t)ks * g.M + m) * g.N + n] = acc[0][i][j][r];
                    } else if constexpr (E == Epi::SwiGlu) {
                        const float v = silu(acc[0][i][j][r]) * acc[NB - 1][i][j][r];
                        reinterpret_cast<T *>(e.out)[(size_t)m * g.N + n] = from_f<T>(v);
                    }
                }
    } else {
        // stage the fp32 tile in LDS once every wave is done with the operand tiles
        __syncthreads();
        float *Cs = reinterpret_cast<float *>(lds);
        constexpr int LDC = BN + 4;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Cs[(wm * WTM + i * 16 + lg * 4 + r) * LDC + wn * WTN + j * 16 + lr] = acc[0][i][j][r];
        __syncthreads();
        if constexpr (E == Epi::Qkv) {
            // rotate-half RoPE: pair (j, j + hd/2) of each head of q and k.
            // First the row metadata, once per tile and in parallel: each row's
            // position and, per head of the tile, where its hd values go (a q row,
            // or a row of a K or V cache).  Then every thread loads the (cos, sin)
            // of all its pairs before its first store, so no load waits on a store.
            const int hd = e.hd, half = hd >> 1, nh = BN / hd;
            int *s_pos = reinterpret_cast<int *>(lds + BM * LDC * 4);
            uint64_t *s_dst = reinterpret_cast<uint64_t *>(lds + BM * LDC * 4 + BM * 4);
            for (int t = tid; t < BM * nh; t += NT) {
                const int r = t / nh, hh = t % nh, m = m0 + r;
                T *dst = nullptr;
                if (m < g.M) {
                    if (hh == 0) s_pos[r] = e.pos ? e.pos[m] : m;
                    const int n = n0 + hh * hd;  // first column of this head
                    if (n < e.n_q) {
                        dst = reinterpret_cast<T *>(e.out) + (size_t)m * e.n_q + n;
                    } else if (e.kv_req) {
                        // one of several KV buffers (batched prefill)
                        const int rq = e.kv_req[m], Hkv = e.n_k / hd;
                        const size_t slab = (size_t)e.kv_cap[rq] * hd;
                        const bool is_k = n < e.n_q + e.n_k;
                        const int kh = is_k ? (n - e.n_q) / hd : (n - e.n_q - e.n_k) / hd;
                        dst = reinterpret_cast<T *>(e.kv_base[rq]) +
                              ((size_t)(e.kv_layer * 2 + (is_k ? 0 : 1)) * Hkv + kh) * slab +
                              (size_t)e.kv_row[m] * hd;
                    } else {
                        // rows from kv_split on go to the second cache (the branch tokens of a fused pass)
                        const bool second = m >= e.kv_split;
                        const int mr = second ? m - e.kv_split : m, cap = second ? e.cap2 : e.cap;
                        if (n < e.n_q + e.n_k) {
                            const int kh = (n - e.n_q) / hd;
                            dst = reinterpret_cast<T *>(second ? e.kc2 : e.kc) + ((size_t)kh * cap + mr) * hd;
                        } else {
                            const int vh = (n - e.n_q - e.n_k) / hd;
                            dst = reinterpret_cast<T *>(second ? e.vc2 : e.vc) + ((size_t)vh * cap + mr) * hd;
                        }
                    }
                }
                s_dst[r * 4 + hh] = reinterpret_cast<uint64_t>(dst);
            }
            __syncthreads();
            // Each item is a run of 8 pairs (j .. j+7 with j + hd/2 ..): its
            // (cos, sin) values and both 8-column runs of the tile row are read
            // in 16-byte vectors and the two runs go out as 16-byte stores
            // (hd/2 is a multiple of 8 for head dims 32, 64 and 128).
            constexpr int RUN = 8, RPR = BN / 2 / RUN, ITEMS = BM * RPR, IT = ITEMS / NT;
            static_assert(IT * NT == ITEMS && BN == 128, "runs per thread");
            float4 cs[IT][RUN / 2];  // (cos, sin) of pairs j + 2q and j + 2q + 1
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int idx = tid + it * NT, r = idx / RPR, c = (idx % RPR) * RUN;
                const int hh = c / half, j = c % half;
                const bool rot = m0 + r < g.M && n0 + hh * hd < e.n_q + e.n_k;
                const float4 *src = reinterpret_cast<const float4 *>(e.rope + (size_t)(rot ? s_pos[r] : 0) * half + j);
#pragma unroll
                for (int q = 0; q < RUN / 2; ++q) cs[it][q] = rot ? src[q] : make_float4(1.f, 0.f, 1.f, 0.f);
            }
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int idx = tid + it * NT, r = idx / RPR, c = (idx % RPR) * RUN;
                const int hh = c / half, j = c % half;
                T *dst = reinterpret_cast<T *>(s_dst[r * 4 + hh]);
                if (!dst) continue;  // row past M
                const float *c1 = Cs + r * LDC + hh * hd + j, *c2 = c1 + half;
                float v1[RUN], v2[RUN];
#pragma unroll
                for (int q = 0; q < RUN / 4; ++q) {
                    const float4 a = reinterpret_cast<const float4 *>(c1)[q], b = reinterpret_cast<const float4 *>(c2)[q];
                    v1[4 * q] = a.x; v1[4 * q + 1] = a.y; v1[4 * q + 2] = a.z; v1[4 * q + 3] = a.w;
                    v2[4 * q] = b.x; v2[4 * q + 1] = b.y; v2[4 * q + 2] = b.z; v2[4 * q + 3] = b.w;
                }
                if (n0 + hh * hd < e.n_q + e.n_k) {
#pragma unroll
                    for (int k = 0; k < RUN; ++k) {
                        const float4 t = cs[it][k / 2];
                        const float co = (k & 1) ? t.z : t.x, si = (k & 1) ? t.w : t.y;
                        const float o1 = v1[k] * co - v2[k] * si, o2 = v2[k] * co + v1[k] * si;
                        v1[k] = o1;
                        v2[k] = o2;
                    }
                }
                store8(dst + j, v1);
                store8(dst + j + half, v2);
            }
        } else if constexpr (E == Epi::Readout) {
            // per readout row: max and sum of exp over each 128 vocab columns of
            // this tile (the partials are [N/128][M] whatever the tile width)
            static_assert(BN % 128 == 0, "readout tiles cover whole 128-column slices");
            for (int r = w; r < BM; r += NW) {
                const int m = m0 + r;
                if (m >= g.M) break;
#pragma unroll
                for (int sub = 0; sub < BN / 128; ++sub) {
                    if (n0 + sub * 128 >= g.N) break;  // past the vocabulary (ragged last tile)
                    const float *cr = Cs + r * LDC + sub * 128;
                    float mx = -INFINITY;
                    for (int c = lane; c < 128; c += 64) mx = fmaxf(mx, cr[c]);
                    mx = wave_max(mx);
                    float s = 0.f;
                    for (int c = lane; c < 128; c += 64) s += __expf(cr[c] - mx);
                    s = wave_sum(s);
                    if (lane == 0) e.ro_part[((size_t)tn * (BN / 128) + sub) * g.M + m] = make_float2(mx, s);
                }
            }
            // candidate-token logits that fall in this tile
            for (int q = tid; q < e.n_gather; q += NT) {
                const int ro = e.g_ro[q], tk = e.g_tok[q];
                if (ro >= m0 && ro < m0 + BM && tk >= n0 && tk < n0 + BN) e.g_logit[q] = Cs[(ro - m0) * LDC + (tk - n0)];
            }
        }
    }
}

// ILV: the refill of each stage goes out one DMA instruction at a time
// between runs of matrix instructions instead of in one burst ahead of them
// (bit-identical results).  With three or more stages the refill has a
// stage of slack and this is faster (799 rows: down 34.8 -> 32.1 us, O 11.0
// -> 10.2 us; down at 512 rows 24.9 -> 23.9 us); with two stages it is
// slower for 192x128 tiles (39.3 -> 41.9 us) and slightly faster for the
// 128x256 gate/up tile (54.6 -> 54.1 us), which turns it on itself.
template <typename T, int BM, int BN, int WM, int WN, int NB, int S, Epi E, int KB = 128, bool ILV = (S >= 3)>
static void launch_gemm(const GemmCall &c, int splits, hipStream_t st) {
    constexpr int BK = KB / sizeof(T);
    GemmArgs<NB> g;
    g.A = c.A;
    for (int q = 0; q < NB; ++q) g.B[q] = c.B[q];
    g.M = c.M;
    g.N = c.N;
    g.K = c.K;
    g.tiles_m = (c.M + BM - 1) / BM;
    g.tiles_n = (c.N + BN - 1) / BN;  // only the readout may leave a ragged last tile
    g.splits = splits;
    g.k_per_split = c.K / splits;
    g.total = g.tiles_m * g.tiles_n * g.splits;
    g.per_xcd = (g.total + 7) / 8;
    g.stagger = c.stagger;
    // With a single row tile no workgroup reads another's B lines (the
    // 28-row LM-head readout: 97 -> 80 us); with several, the non-temporal
    // hint evicts lines the other row tiles still need (every GEMM of the
    // passes 5-35% slower).  Only the readout GEMM uses it: in the other
    // one-tile GEMMs the per-load choice cost more than it saved.
    g.b_once = g.tiles_m == 1;
    static_assert(BK > 0, "");
    EpiArgs e;
    e.x = c.x;
    e.part = c.part;
    e.out = c.out;
    e.kc = c.kc;
    e.vc = c.vc;
    e.cap = c.cap;
    e.kc2 = c.kc2;
    e.vc2 = c.vc2;
    e.cap2 = c.cap2;
    e.kv_split = c.kc2 ? c.kv_split : c.M;
    e.kv_req = c.kv_req;
    e.kv_row = c.kv_row;
    e.kv_cap = c.kv_cap;
    e.kv_base = c.kv_base;
    e.kv_layer = c.kv_layer;
    e.n_q = c.n_q;
    e.n_k = c.n_k;
    e.hd = c.hd;
    e.pos = c.pos;
    e.rope = c.rope;
    e.ro_part = c.ro_part;
    e.g_tok = c.g_tok;
    e.g_ro = c.g_ro;
    e.n_gather = c.n_gather;
    e.g_logit = c.g_logit;
    const int shmem = GemmLds<T, BM, BN, NB, E, KB>::bytes(S);
    auto kern = k_gemm<T, BM, BN, WM, WN, NB, S, E, KB, ILV>;
    static bool attr_set = false;  // one model per thread at a time; a repeated set is harmless
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  shmem);
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(g.per_xcd * 8), dim3(WM * WN * 64), shmem, st, g, e);
}

enum class Reg { Small, Medium, Big };
static Reg regime(int M) { return M >= 384 ? Reg::Big : (M > 48 ? Reg::Medium : Reg::Small); }

// split-K for an epilogue that adds into the residual stream: enough
// workgroups for the chip, partial sums within the caller's buffer
// (a split grid that would need a second round of workgroups is not used: at
// 2,048 rows the O projection's 192 tiles took 37.9 us in two splits against
// 29.8 us unsplit at 2,106 rows)
static int pick_splits(const GemmCall &c, int tiles, int BK) {
    if (tiles >= 200) return 1;
    int best = 1;
    for (int s = 2; s <= 8; ++s) {
        if (tiles * s > 256) break;
        if (c.K % (s * BK) || c.K / s < 2 * BK || (size_t)s * c.M * c.N > c.part_cap) continue;
        best = s;
        if (tiles * s >= 240) break;
    }
    return best;
}

// Residual GEMMs write fp32 partial sums (split-K when the tile count is
// small), then one kernel per row adds them into the residual stream and
// writes the next RMSNorm's bf16 input.
template <typename T, int BM, int BN, int WM, int WN, int S, int KB = 128>
static void gemm_resid_cfg(const GemmCall &c, hipStream_t st, int splits = 0) {
    constexpr int BK = KB / sizeof(T);
    const int tiles = (c.M + BM - 1) / BM * (c.N / BN);
    const int s = splits > 0 ? splits : pick_splits(c, tiles, BK);
    launch_gemm<T, BM, BN, WM, WN, 1, S, Epi::Partial, KB>(c, s, st);
    resid_norm(c.dt, c.part, s, c.M, c.N, c.x, c.norm_w, c.eps, c.h_out, st);
}

// Tile shapes per row-count regime, chosen from measurements at the 1.5B
// widths (d 1536, FFN 8960, vocabulary 151936) on MI355X.  fp32 models (the
// tiny configuration) use 32-row tiles with 256-byte k-tiles throughout.
// k-order stagger of the row tiles (GemmArgs::stagger) per GEMM, measured
// with cold weights at the 1.5B widths: QKV (9 to 25 row tiles per weight
// slab) 3 stages (13.4 -> 11.7 us at 287 rows, 16.3 -> 14.4 us at 799);
// gate/up and down 1 stage (4-7% and 2-3% at 287-799 rows); the O
// projection none (1 stage is 3% slower at 799 rows).  In the 16,384-token
// 7B prefill and the 64-request batch, gate/up gains 1.5-3% and the others
// stay within 1%.
static int stagger_for(const GemmCall &c) {
    switch (c.epi) {
        case Epi::Qkv: return 3;
        case Epi::SwiGlu: return 1;
        case Epi::Resid: return c.K >= 4096 ? 1 : 0;
        default: return 0;
    }
}

template <typename T> static bool gemm_t(const GemmCall &c0, hipStream_t st) {
    GemmCall c = c0;
    if (sizeof(T) == 2) c.stagger = stagger_for(c0);
    constexpr int KB = sizeof(T) == 2 ? 128 : 256;
    constexpr int BK = KB / sizeof(T);
    if (c.M <= 0 || c.N % 128 || c.K % BK) return false;
    if constexpr (sizeof(T) == 4) {
        switch (c.epi) {
            case Epi::Qkv:
                if (128 % c.hd) return false;
                launch_gemm<T, 32, 128, 1, 4, 1, 4, Epi::Qkv, KB>(c, 1, st);
                return true;
            case Epi::Readout: launch_gemm<T, 32, 128, 1, 4, 1, 4, Epi::Readout, KB>(c, 1, st); return true;
            case Epi::Resid: gemm_resid_cfg<T, 32, 128, 1, 4, 4, KB>(c, st); return true;
            case Epi::SwiGlu: launch_gemm<T, 32, 64, 1, 4, 2, 4, Epi::SwiGlu, KB>(c, 1, st); return true;
            case Epi::Partial: return false;
        }
        return false;
    } else {
        const Reg rg = regime(c.M);
        switch (c.epi) {
            case Epi::Qkv:
                if (128 % c.hd) return false;
                // many rows: 256x128 tiles once they alone fill the chip (64 x 1,024-token
                // batched prefill: 0.69 against 0.80 ms per layer), or where 128x128 would
                // need a second round and 256x128 fits one
                if (c.M > 1024 && ((c.M + 255) / 256 * (c.N / 128) >= 240 ||
                                   ((c.M + 127) / 128 * (c.N / 128) > 256 && (c.M + 255) / 256 * (c.N / 128) <= 256))) {
                    launch_gemm<T, 256, 128, 2, 4, 1, 3, Epi::Qkv>(c, 1, st);
                } else if (c.M > 1024) {
                    launch_gemm<T, 128, 128, 2, 4, 1, 3, Epi::Qkv>(c, 1, st);
                } else {
                    // 32-row tiles while they fit one round of workgroups; 64-row
                    // tiles (8 waves) once 32 rows would need a second round
                    // (799 rows: 15.5 us against 17.8 us)
                    const int tn = c.N / 128;
                    if ((c.M + 31) / 32 * tn > 256 && (c.M + 63) / 64 * tn <= 256)
                        launch_gemm<T, 64, 128, 2, 4, 1, 4, Epi::Qkv>(c, 1, st);
                    // 128-row tiles where 64-row ones would need a second round and these
                    // fit one (7B widths, 668 rows: 35.9 against 53.3 us with 32-row tiles)
                    else if ((c.M + 63) / 64 * tn > 256 && (c.M + 127) / 128 * tn <= 256)
                        launch_gemm<T, 128, 128, 2, 4, 1, 3, Epi::Qkv>(c, 1, st);
                    else launch_gemm<T, 32, 128, 1, 4, 1, 4, Epi::Qkv>(c, 1, st);
                }
                return true;
            case Epi::Readout:
                if (rg == Reg::Small) launch_gemm<T, 32, 128, 1, 4, 1, 4, Epi::Readout>(c, 1, st);
                else if (rg == Reg::Medium) launch_gemm<T, 64, 128, 2, 2, 1, 4, Epi::Readout>(c, 1, st);
                // many readout rows: 256 vocab columns per tile (1,792 rows: 1.31 against 1.78 ms)
                else if (c.M > 1024) launch_gemm<T, 128, 256, 2, 4, 1, 2, Epi::Readout>(c, 1, st);
                else launch_gemm<T, 128, 128, 2, 4, 1, 3, Epi::Readout>(c, 1, st);
                return true;
            case Epi::Resid:
                if (rg == Reg::Small) gemm_resid_cfg<T, 32, 128, 1, 4, 4>(c, st);
                // many rows: 256x256 tiles (half the operand bytes per flop of 128x128)
                // once they alone fill the chip (65,536 rows: O 0.31 against 0.48 ms,
                // down 1.44 against 2.20 ms)
                else if (c.M > 1024 && (c.M + 255) / 256 * (c.N / 256) >= 240 && c.N % 256 == 0)
                    gemm_resid_cfg<T, 256, 256, 2, 4, 2>(c, st);
                else if (c.K < 4096 && c.M > 1024) gemm_resid_cfg<T, 128, 128, 2, 4, 3>(c, st);
                else if (c.K < 4096) {
                    // 96-row tiles where 64-row ones would need a second round of
                    // workgroups and 96-row ones fit one (799 rows: 17.4 us against 18.3 us
                    // with the residual kernel)
                    // Unsplit 128x128 tiles where 96x64 ones would need a second round and
                    // these fit one (7B widths, 668 rows: 37.9 against 49.9 us with 64x64).
                    const int tn = c.N / 64;
                    if ((c.M + 63) / 64 * tn > 256 && (c.M + 95) / 96 * tn <= 256)
                        gemm_resid_cfg<T, 96, 64, 2, 2, 4>(c, st);
                    else if ((c.M + 95) / 96 * tn > 256 && (c.M + 127) / 128 * (c.N / 128) <= 256)
                        gemm_resid_cfg<T, 128, 128, 2, 4, 3>(c, st, 1);
                    else gemm_resid_cfg<T, 64, 64, 2, 2, 4>(c, st);
                }
                // Long K (the down projection): 256x256 tiles in 4 K-splits once that
                // gives 160 to 256 workgroups (7B widths, 668 rows: 118 against 200 us
                // with 160x128 tiles in 2 splits, residual kernel included).
                else if (c.N % 256 == 0 && c.K % (4 * BK) == 0 && c.K / 4 >= 2048 &&
                         (c.M + 255) / 256 * (c.N / 256) * 4 >= 160 && (c.M + 255) / 256 * (c.N / 256) * 4 <= 256 &&
                         (size_t)4 * c.M * c.N <= c.part_cap)
                    gemm_resid_cfg<T, 256, 256, 2, 4, 2>(c, st, 4);
                // 160-row tiles where they need fewer row tiles than 128-row ones
                // (799 rows: 5 instead of 7, so the split-K grid fits one round)
                else if (rg == Reg::Big && c.M <= 1024 && (c.M + 159) / 160 < (c.M + 127) / 128)
                    gemm_resid_cfg<T, 160, 128, 2, 2, 4>(c, st);
                else gemm_resid_cfg<T, 128, 128, 2, 4, 3>(c, st);
                return true;
            case Epi::SwiGlu: {
                // 128x160 (gate/up pair) when it covers the product in one round of
                // workgroups and 128x128 does not; 128x128 otherwise, whose second
                // round is still cheaper per tile than any smaller tile's rounds
                const int rows = (c.M + 127) / 128;
                if (rg == Reg::Small) launch_gemm<T, 32, 64, 1, 4, 2, 4, Epi::SwiGlu>(c, 1, st);
                // many rows: 256-row tiles (2,048 rows: 115 against 120 us; 65,536: 2.76 against 3.12 ms)
                else if (c.M > 1024) launch_gemm<T, 256, 128, 2, 4, 2, 2, Epi::SwiGlu>(c, 1, st);
                // 192-row tiles where 128-row ones would need a second round and these
                // fit one: as many operand bytes per workgroup as 128x160, in 8 waves
                // instead of 4 (512 rows: 39.1 against 41.7 us with cold weights)
                else if (rows * (c.N / 128) > 256 && (c.M + 191) / 192 * (c.N / 128) <= 256)
                    launch_gemm<T, 192, 128, 2, 4, 2, 2, Epi::SwiGlu>(c, 1, st);
                else if (rows * (c.N / 128) > 256 && c.N % 160 == 0 && rows * (c.N / 160) <= 256)
                    launch_gemm<T, 128, 160, 2, 2, 2, 2, Epi::SwiGlu>(c, 1, st);
                // 128x256 when that fits one round (each workgroup reads its rows of the
                // activations once for what two 128x128 tiles in two rounds would do;
                // 799 rows: 54.2 against 58.6 us with cold weights, 51.9 against 53.0 us
                // in the single pass)
                else if (rows * (c.N / 128) > 256 && c.N % 256 == 0 && rows * (c.N / 256) <= 256)
                    launch_gemm<T, 128, 256, 2, 4, 2, 2, Epi::SwiGlu, 128, true>(c, 1, st);
                // 256-row tiles when 128-row ones would take more than two rounds (7B
                // widths, 668 rows: 211 against 236 us)
                else if (rows * (c.N / 128) > 2 * 256)
                    launch_gemm<T, 256, 128, 2, 4, 2, 2, Epi::SwiGlu>(c, 1, st);
                else launch_gemm<T, 128, 128, 2, 4, 2, 3, Epi::SwiGlu>(c, 1, st);
                return true;
            }
            case Epi::Partial:
                return false;  // chosen internally by Resid
        }
        return false;
    }
}

bool gemm(const GemmCall &c, hipStream_t st) {
    return c.dt == PCD_DT_F32 ? gemm_t<float>(c, st) : gemm_t<bf16_t>(c, st);
}
int gemm_k_tile(int dt) { return dt == PCD_DT_F32 ? 64 : 64; }

// ---------------------------------------------------------------------------
// embedding gather, RMSNorm, split-K reduction
// ---------------------------------------------------------------------------
// x[t] = E[tok[t]] (fp32) and h[t] = rmsnorm(x[t]) * w (dt): the first
// layer's normalised input comes out of the embedding gather.
template <typename T>
__global__ __launch_bounds__(256) void k_embed(const int32_t *tok, const T *E, int32_t d, float *x, const float *w,
                                               float eps, T *h) {
    __shared__ float red[4];
    const int t = blockIdx.x;
    const T *row = E + (size_t)tok[t] * d;
    float ss = 0.f;
    for (int j = threadIdx.x; j < d; j += 256) {
        const float v = to_f(row[j]);
        x[(size_t)t * d + j] = v;
        ss += v * v;
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d + eps);
    for (int j = threadIdx.x; j < d; j += 256) h[(size_t)t * d + j] = from_f<T>(to_f(row[j]) * inv * w[j]);
}

// The same for d = 512 * NE: the row and the norm weight are loaded once, up
// front, as pairs, so a row costs one memory round trip.
template <typename T, int NE>
__global__ __launch_bounds__(256) void k_embed_n(const int32_t *tok, const T *E, float *x, const float *w, float eps,
                                                 T *h) {
    constexpr int D = 512 * NE;
    __shared__ float red[4];
    const int t = blockIdx.x, tid = threadIdx.x;
    const T *row = E + (size_t)tok[t] * D;
    float2 v[NE], wv[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int j = 2 * (tid + 256 * i);
        v[i] = make_float2(to_f(row[j]), to_f(row[j + 1]));
        wv[i] = reinterpret_cast<const float2 *>(w)[tid + 256 * i];
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        reinterpret_cast<float2 *>(x + (size_t)t * D)[tid + 256 * i] = v[i];
        ss += v[i].x * v[i].x + v[i].y * v[i].y;
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)D + eps);
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        T *hp = h + (size_t)t * D + 2 * (tid + 256 * i);
        hp[0] = from_f<T>(v[i].x * inv * wv[i].x);
        hp[1] = from_f<T>(v[i].y * inv * wv[i].y);
    }
}

void embed(int dt, const int32_t *tok, int32_t T, const void *E, int32_t d, float *x, const float *w, float eps,
           void *h, hipStream_t st) {
    if (T <= 0) return;
    if (dt != PCD_DT_F32 && d == 1536)
        hipLaunchKernelGGL((k_embed_n<bf16_t, 3>), dim3(T), dim3(256), 0, st, tok, (const bf16_t *)E, x, w, eps,
                           (bf16_t *)h);
    else if (dt != PCD_DT_F32 && d == 3584)
        hipLaunchKernelGGL((k_embed_n<bf16_t, 7>), dim3(T), dim3(256), 0, st, tok, (const bf16_t *)E, x, w, eps,
                           (bf16_t *)h);
    else if (dt == PCD_DT_F32)
        hipLaunchKernelGGL(k_embed<float>, dim3(T), dim3(256), 0, st, tok, (const float *)E, d, x, w, eps, (float *)h);
    else
        hipLaunchKernelGGL(k_embed<bf16_t>, dim3(T), dim3(256), 0, st, tok, (const bf16_t *)E, d, x, w, eps,
                           (bf16_t *)h);
}

template <typename T>
__global__ void k_rmsnorm(const float *x, const int32_t *rows, int32_t d, const float *w, float eps, T *out) {
    __shared__ float red[4];
    const int i = blockIdx.x;
    const float *xr = x + (size_t)(rows ? rows[i] : i) * d;
    float s = 0.f;
    for (int j = threadIdx.x; j < d; j += 256) s += xr[j] * xr[j];
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    const float tot = red[0] + red[1] + red[2] + red[3];
    const float inv = 1.0f / sqrtf(tot / (float)d + eps);
    for (int j = threadIdx.x; j < d; j += 256) out[(size_t)i * d + j] = from_f<T>(xr[j] * inv * w[j]);
}

// The same for d = 512 * NE, every load of the row up front.
template <typename T, int NE>
__global__ __launch_bounds__(256) void k_rmsnorm_n(const float *x, const int32_t *rows, const float *w, float eps,
                                                   T *out) {
    constexpr int D = 512 * NE;
    __shared__ float red[4];
    const int i = blockIdx.x, tid = threadIdx.x;
    const float2 *xr = reinterpret_cast<const float2 *>(x + (size_t)(rows ? rows[i] : i) * D);
    float2 v[NE], wv[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        v[e] = xr[tid + 256 * e];
        wv[e] = reinterpret_cast<const float2 *>(w)[tid + 256 * e];
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) s += v[e].x * v[e].x + v[e].y * v[e].y;
    s = wave_sum(s);
    if ((tid & 63) == 0) red[tid >> 6] = s;
    __syncthreads();
    const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)D + eps);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        T *op = out + (size_t)i * D + 2 * (tid + 256 * e);
        op[0] = from_f<T>(v[e].x * inv * wv[e].x);
        op[1] = from_f<T>(v[e].y * inv * wv[e].y);
    }
}

void rmsnorm(int dt, const float *x, const int32_t *rows, int32_t n, int32_t d, const float *w, float eps, void *out,
             hipStream_t st) {
    if (n <= 0) return;
    if (dt != PCD_DT_F32 && d == 1536)
        hipLaunchKernelGGL((k_rmsnorm_n<bf16_t, 3>), dim3(n), dim3(256), 0, st, x, rows, w, eps, (bf16_t *)out);
    else if (dt != PCD_DT_F32 && d == 3584)
        hipLaunchKernelGGL((k_rmsnorm_n<bf16_t, 7>), dim3(n), dim3(256), 0, st, x, rows, w, eps, (bf16_t *)out);
    else if (dt == PCD_DT_F32)
        hipLaunchKernelGGL(k_rmsnorm<float>, dim3(n), dim3(256), 0, st, x, rows, d, w, eps, (float *)out);
    else hipLaunchKernelGGL(k_rmsnorm<bf16_t>, dim3(n), dim3(256), 0, st, x, rows, d, w, eps, (bf16_t *)out);
}

// One workgroup per row m: x[m] += sum over s of part[s][m] (s in increasing
// order, so the result does not depend on scheduling), then, if w is given,
// h[m] = rmsnorm(x[m]) * w as the next GEMM's input.  SMAX >= splits: the
// loads of every split are issued together (splits beyond the real count
// re-read the last one and add nothing), so a row costs one memory round
// trip rather than one per split.  VEC2: N is a multiple of 512 and at most
// 8192, each thread moves float2s.
template <typename T, int SMAX, bool VEC2>
__global__ __launch_bounds__(256) void k_resid_norm(const float *__restrict__ part, int32_t splits, int32_t M,
                                                    int32_t N, float *__restrict__ x, const float *__restrict__ w,
                                                    float eps, T *__restrict__ h) {
    __shared__ float red[4];
    const int m = blockIdx.x, tid = threadIdx.x;
    float *xr = x + (size_t)m * N;
    const size_t pstride = (size_t)M * N;
    const float *prow = part + (size_t)m * N;
    float ss = 0.f;
    if constexpr (VEC2) {
        constexpr int MAXE = 16;
        const int ne = N / 512;
        float2 acc[MAXE];
#pragma unroll
        for (int i = 0; i < MAXE; ++i) {
            if (i >= ne) break;
            const int j = tid + 256 * i;
            float2 v = reinterpret_cast<const float2 *>(xr)[j];
            float2 pv[SMAX];
#pragma unroll
            for (int s = 0; s < SMAX; ++s)
                pv[s] = reinterpret_cast<const float2 *>(prow + (size_t)min(s, splits - 1) * pstride)[j];
#pragma unroll
            for (int s = 0; s < SMAX; ++s)
                if (s < splits) {
                    v.x += pv[s].x;
                    v.y += pv[s].y;
                }
            acc[i] = v;
            reinterpret_cast<float2 *>(xr)[j] = v;
            ss += v.x * v.x + v.y * v.y;
        }
        if (!w) return;
        ss = wave_sum(ss);
        if ((tid & 63) == 0) red[tid >> 6] = ss;
        __syncthreads();
        const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)N + eps);
#pragma unroll
        for (int i = 0; i < MAXE; ++i) {
            if (i >= ne) break;
            const int j = 2 * (tid + 256 * i);
            h[(size_t)m * N + j] = from_f<T>(acc[i].x * inv * w[j]);
            h[(size_t)m * N + j + 1] = from_f<T>(acc[i].y * inv * w[j + 1]);
        }
    } else {
        for (int j = tid; j < N; j += 256) {
            float v = xr[j];
            float pv[SMAX];
#pragma unroll
            for (int s = 0; s < SMAX; ++s) pv[s] = prow[(size_t)min(s, splits - 1) * pstride + j];
#pragma unroll
            for (int s = 0; s < SMAX; ++s)
                if (s < splits) v += pv[s];
            xr[j] = v;
            ss += v * v;
        }
        if (!w) return;
        ss = wave_sum(ss);
        if ((tid & 63) == 0) red[tid >> 6] = ss;
        __syncthreads();
        const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)N + eps);
        for (int j = tid; j < N; j += 256) h[(size_t)m * N + j] = from_f<T>(xr[j] * inv * w[j]);
    }
}

// The same for N = 512 * NE, one wave per row: each lane loads its 4-float
// slices of the row, of every split's partial and of the norm weight up
// front, so a row costs one memory round trip (loading w only after the
// reduction cost 1.5-2.7 us per launch at 799 rows of 1536), and the row's
// sum of squares is a wave reduction (no LDS, no barrier; 0.5 us faster per
// launch than a workgroup per row).  Four rows per workgroup.
template <typename T, int SMAX, int NE>
__global__ __launch_bounds__(256) void k_resid_norm_n(const float *__restrict__ part, int32_t splits, int32_t M,
                                                      float *__restrict__ x, const float *__restrict__ w, float eps,
                                                      T *__restrict__ h) {
    constexpr int N = 512 * NE, NV = 2 * NE;  // float4 slices per lane
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    float *xr = x + (size_t)m * N;
    const size_t pstride = (size_t)M * N;
    const float *prow = part + (size_t)m * N;
    float4 v[NV], wv[NV], pv[NV][SMAX];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = lane + 64 * i;
        v[i] = reinterpret_cast<const float4 *>(xr)[j];
        if (w) wv[i] = reinterpret_cast<const float4 *>(w)[j];
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
            pv[i][s] = reinterpret_cast<const float4 *>(prow + (size_t)min(s, splits - 1) * pstride)[j];
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
            if (s < splits) {
                v[i].x += pv[i][s].x;
                v[i].y += pv[i][s].y;
                v[i].z += pv[i][s].z;
                v[i].w += pv[i][s].w;
            }
        reinterpret_cast<float4 *>(xr)[lane + 64 * i] = v[i];
        ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    }
    if (!w) return;
    const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)N + eps);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = lane + 64 * i;
        const float4 o = make_float4(v[i].x * inv * wv[i].x, v[i].y * inv * wv[i].y, v[i].z * inv * wv[i].z,
                                     v[i].w * inv * wv[i].w);
        if constexpr (sizeof(T) == 2) {
            const uint32_t a = __builtin_bit_cast(uint16_t, from_f<T>(o.x));
            const uint32_t b = __builtin_bit_cast(uint16_t, from_f<T>(o.y));
            const uint32_t c = __builtin_bit_cast(uint16_t, from_f<T>(o.z));
            const uint32_t d = __builtin_bit_cast(uint16_t, from_f<T>(o.w));
            reinterpret_cast<uint2 *>(h + (size_t)m * N)[j] = make_uint2(a | (b << 16), c | (d << 16));
        } else {
            reinterpret_cast<float4 *>(h + (size_t)m * N)[j] = o;
        }
    }
}

// The same for N = 512 * NE, one workgroup per row (2 values per thread per
// 512 columns): for the wider rows (3584) one wave per row would hold every
// split's slice of the row in a lane's registers, up to 512 of them with
// spills at 8 splits.  Every load still goes out before the first use.
template <typename T, int SMAX, int NE>
__global__ __launch_bounds__(256) void k_resid_norm_wg(const float *__restrict__ part, int32_t splits, int32_t M,
                                                      float *__restrict__ x, const float *__restrict__ w, float eps,
                                                      T *__restrict__ h) {
    constexpr int N = 512 * NE;
    __shared__ float red[4];
    const int m = blockIdx.x, tid = threadIdx.x;
    float *xr = x + (size_t)m * N;
    const size_t pstride = (size_t)M * N;
    const float *prow = part + (size_t)m * N;
    float2 v[NE], wv[NE], pv[NE][SMAX];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int j = tid + 256 * i;
        v[i] = reinterpret_cast<const float2 *>(xr)[j];
        if (w) wv[i] = reinterpret_cast<const float2 *>(w)[j];
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
            pv[i][s] = reinterpret_cast<const float2 *>(prow + (size_t)min(s, splits - 1) * pstride)[j];
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
            if (s < splits) {
                v[i].x += pv[i][s].x;
                v[i].y += pv[i][s].y;
            }
        reinterpret_cast<float2 *>(xr)[tid + 256 * i] = v[i];
        ss += v[i].x * v[i].x + v[i].y * v[i].y;
    }
    if (!w) return;
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)N + eps);
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int j = tid + 256 * i;
        T *hp = h + (size_t)m * N + 2 * j;
        if constexpr (sizeof(T) == 2) {
            const uint32_t lo = __builtin_bit_cast(uint16_t, from_f<T>(v[i].x * inv * wv[i].x));
            const uint32_t hi = __builtin_bit_cast(uint16_t, from_f<T>(v[i].y * inv * wv[i].y));
            *reinterpret_cast<uint32_t *>(hp) = lo | (hi << 16);
        } else {
            *reinterpret_cast<float2 *>(hp) = make_float2(v[i].x * inv * wv[i].x, v[i].y * inv * wv[i].y);
        }
    }
}

template <typename T, int SMAX>
static void resid_norm_t(const float *part, int32_t splits, int32_t M, int32_t N, float *x, const float *w, float eps,
                         void *h, hipStream_t st) {
    if (N == 1536)
        hipLaunchKernelGGL((k_resid_norm_n<T, SMAX, 3>), dim3((M + 3) / 4), dim3(256), 0, st, part, splits, M, x, w, eps, (T *)h);
    else if (N == 3584)
        hipLaunchKernelGGL((k_resid_norm_wg<T, SMAX, 7>), dim3(M), dim3(256), 0, st, part, splits, M, x, w, eps, (T *)h);
    else if (N % 512 == 0 && N <= 8192)
        hipLaunchKernelGGL((k_resid_norm<T, SMAX, true>), dim3(M), dim3(256), 0, st, part, splits, M, N, x, w, eps,
                           (T *)h);
    else
        hipLaunchKernelGGL((k_resid_norm<T, SMAX, false>), dim3(M), dim3(256), 0, st, part, splits, M, N, x, w, eps,
                           (T *)h);
}
template <typename T>
static void resid_norm_s(const float *part, int32_t splits, int32_t M, int32_t N, float *x, const float *w, float eps,
                         void *h, hipStream_t st) {
    if (splits <= 1) resid_norm_t<T, 1>(part, splits, M, N, x, w, eps, h, st);
    else if (splits <= 2) resid_norm_t<T, 2>(part, splits, M, N, x, w, eps, h, st);
    else if (splits <= 4) resid_norm_t<T, 4>(part, splits, M, N, x, w, eps, h, st);
    else resid_norm_t<T, 8>(part, splits, M, N, x, w, eps, h, st);
}

void resid_norm(int dt, const float *part, int32_t splits, int32_t M, int32_t N, float *x, const float *w, float eps,
                void *h, hipStream_t st) {
    if (M <= 0) return;
    if (dt == PCD_DT_F32) resid_norm_s<float>(part, splits, M, N, x, w, eps, h, st);
    else resid_norm_s<bf16_t>(part, splits, M, N, x, w, eps, h, st);
}

// ---------------------------------------------------------------------------
// Attention over KV caches: 64 query rows per workgroup (16 per wave); query
// rows are (token, head within the KV group) pairs, so the heads of a GQA
// group share every staged K/V tile.  Key tiles of 64 are double-buffered:
// while the matrix cores work on tile i from LDS, tile i+1 is already on its
// way from global memory into registers.  S^T = K Q^T on the matrix cores so
// that each lane holds 4 keys of one query row; online softmax in base 2 with
// the row statistics reduced across the four lane groups; O += P V on the
// matrix cores.
//
// A block first walks its prefix keys [key0, key1) (causal for prefill), then
// -- branch tokens only -- the branch keys [sfx_lo, sfx_hi) of the fields its
// rows belong to, masked to each row's scaffold up to itself and its trie
// ancestors.  One split: the block writes the final output; several: it
// writes (max, sum, unnormalised O) partials for the merge kernel.
// ---------------------------------------------------------------------------
// Visibility of branch key k to branch token t, from t's field start fs,
// scaffold length ns and its trie chain (itself, parent, ...): a scaffold key
// is seen by every trie token of its field and by the scaffold tokens after
// it; a trie key only by itself and its descendants.  The first 8 links of
// the chain come from the plan's chain table (two independent loads) and sit
// in registers; longer chains continue through the parent links in memory.
struct RowVis {
    int t, fs, ns, nch, tail;  // tail: parent of the last stored link (-1: chain complete)
    int chain[8];
    bool trie;
};
__device__ __forceinline__ void row_vis_init(RowVis &v, const AttnCall &c, int t) {
    v.t = t;
    v.fs = c.fs[t];
    v.ns = c.nsc[t];
    v.trie = t >= v.fs + v.ns;
    v.nch = 0;
    v.tail = -1;
    if (v.trie) {
        const int4 a = c.chain[2 * t], b = c.chain[2 * t + 1];
        const int ch[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v.chain[i] = ch[i];
            if (ch[i] >= 0) v.nch = i + 1;
        }
        v.tail = v.chain[7] >= 0 ? c.par[v.chain[7]] : -1;
    }
}
__device__ __forceinline__ bool row_vis_sees(const RowVis &v, const AttnCall &c, int k) {
    if (k < v.fs) return false;
    if (k < v.fs + v.ns) return v.trie || k <= v.t;
    if (!v.trie) return false;
    bool hit = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) hit |= (i < v.nch && v.chain[i] == k);
    if (hit || v.tail < 0) return hit;
    int a = v.tail;
    while (a > k) a = c.par[a];
    return a == k;
}

// Output of one attention workgroup: O row 4*lg + r of wave w, normalised
// when the row has no other split, else (unnormalised O, max, sum) partials
// for the merge kernel.  l is the row's full sum (replicated over lg).
template <typename T, int HD>
__device__ __forceinline__ void attn_write(const AttnCall &c, const AttnBlock &blk, const f32x4 (&o)[HD / 16],
                                           float m_run, float l_run, int w, int lr, int lg) {
    constexpr int CF = HD / 16;
    const int Hq = c.n_heads, grp = Hq / c.n_kv_heads;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int qi = lg * 4 + r;
        const float lq = __shfl(l_run, qi);
        const float mq = __shfl(m_run, qi);
        if (w * 16 + qi >= blk.nrows) continue;
        const int row = blk.row0 + w * 16 + qi;
        const int t = row / grp, h = blk.g * grp + row % grp;
        if (blk.causal && blk.qoff + t < blk.key0) continue;  // causal row with no key in this split
        if (c.tok_splits[t] <= 1) {
            T *out = reinterpret_cast<T *>(c.out) + ((size_t)t * Hq + h) * HD;
            const float inv = 1.0f / lq;
#pragma unroll
            for (int j = 0; j < CF; ++j) out[j * 16 + lr] = from_f<T>(o[j][r] * inv);
        } else {
            const size_t pi = ((size_t)blk.split * c.n_tokens + t) * Hq + h;
            float *po = c.part_o + pi * HD;
#pragma unroll
            for (int j = 0; j < CF; ++j) po[j * 16 + lr] = o[j][r];
            if (lr == 0) c.part_ml[pi] = make_float2(mq, lq);
        }
    }
}

// The same for an O whose lane holds its own query row lr, columns
// 16 j + 4 lg .. + 3 (P*V with V's fragment as the first operand): four
// adjacent outputs per store, and the row's (max, sum) already in the lane.
template <typename T, int HD>
__device__ __forceinline__ void attn_write_rows(const AttnCall &c, const AttnBlock &blk, const f32x4 (&o)[HD / 16],
                                                float m_run, float l_run, int w, int lr, int lg) {
    constexpr int CF = HD / 16;
    const int Hq = c.n_heads, grp = Hq / c.n_kv_heads;
    if (w * 16 + lr >= blk.nrows) return;
    const int row = blk.row0 + w * 16 + lr;
    const int t = row / grp, h = blk.g * grp + row % grp;
    if (blk.causal && blk.qoff + t < blk.key0) return;  // causal row with no key in this split
    if (c.tok_splits[t] <= 1) {
        T *out = reinterpret_cast<T *>(c.out) + ((size_t)t * Hq + h) * HD + 4 * lg;
        const float inv = 1.0f / l_run;
#pragma unroll
        for (int j = 0; j < CF; ++j) {
            const float2v_t lo = {o[j][0] * inv, o[j][1] * inv}, hi = {o[j][2] * inv, o[j][3] * inv};
            const uint2 u = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2v_t)),
                             __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2v_t))};
            *reinterpret_cast<uint2 *>(out + j * 16) = u;
        }
    } else {
        const size_t pi = ((size_t)blk.split * c.n_tokens + t) * Hq + h;
        float *po = c.part_o + pi * HD + 4 * lg;
#pragma unroll
        for (int j = 0; j < CF; ++j) *reinterpret_cast<f32x4 *>(po + j * 16) = o[j];
        if (lg == 0) c.part_ml[pi] = make_float2(m_run, l_run);
    }
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn(AttnCall c) {
    constexpr int KT = 64;
    constexpr int KPAD = 16 / sizeof(T);
    constexpr int LDKS = HD + KPAD;   // K tile row stride
    constexpr int LDV = KT + KPAD;    // V^T row stride
    constexpr int HS = HD / 32;       // k-steps of Q.K
    constexpr int CF = HD / 16;       // output column fragments
    constexpr int CH = 16 / sizeof(T);
    constexpr int CHUNKS = KT * HD / CH;
    constexpr int PER_T = CHUNKS / 256;  // 16-byte chunks per thread per tile (K and V each)
    static_assert(PER_T * 256 == CHUNKS, "tile / thread mismatch");
    extern __shared__ __attribute__((aligned(16))) char attn_lds[];
    T *Ks0 = reinterpret_cast<T *>(attn_lds);
    T *Vt0 = Ks0 + KT * LDKS;
    T *Ks1 = Vt0 + HD * LDV;
    T *Vt1 = Ks1 + KT * LDKS;

    const AttnBlock blk = c.blocks[blockIdx.x];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
    const int Hq = c.n_heads, Hkv = c.n_kv_heads, grp = Hq / Hkv;
    const int P = c.req_stride[blk.req];  // slab stride (the buffer's token capacity)
    const T *kvbase = reinterpret_cast<const T *>(c.req_kv[blk.req]);
    const T *Kg = kvbase + ((size_t)c.layer * 2 * Hkv + blk.g) * (size_t)P * HD;
    const T *Vg = kvbase + ((size_t)c.layer * 2 * Hkv + Hkv + blk.g) * (size_t)P * HD;
    const T *Kb = reinterpret_cast<const T *>(c.kb) + (size_t)blk.g * c.cap * HD;
    const T *Vb = reinterpret_cast<const T *>(c.vb) + (size_t)blk.g * c.cap * HD;
    const T *Q = reinterpret_cast<const T *>(c.q);
    const float qscale = LOG2E / sqrtf((float)HD);

    // this lane's query row (B operand of S^T) and its token
    const bool row_ok = (w * 16 + lr) < blk.nrows;
    const int rr = row_ok ? blk.row0 + w * 16 + lr : blk.row0;
    const int tq = rr / grp, hq = blk.g * grp + rr % grp;
    Frag<T> qf[HS];
#pragma unroll
    for (int s = 0; s < HS; ++s) ld8(qf[s], Q + ((size_t)tq * Hq + hq) * HD + s * 32 + lg * 8);
    const int kend_row = blk.causal ? min(blk.qoff + tq + 1, blk.key1) : blk.key1;

    int kmax = blk.key1;
    if (blk.causal) {
        const int last = blk.qoff + (blk.row0 + blk.nrows - 1) / grp + 1;
        kmax = last < kmax ? last : kmax;
    }
    const int n_pre = kmax > blk.key0 ? (kmax - blk.key0 + KT - 1) / KT : 0;
    const int n_sfx = blk.sfx_hi > blk.sfx_lo ? (blk.sfx_hi - blk.sfx_lo + KT - 1) / KT : 0;
    const int n_tiles = n_pre + n_sfx;
    RowVis vis{};
    if (n_sfx > 0) row_vis_init(vis, c, tq - c.branch0);

    // K chunks: 16 consecutive threads cover one key row (coalesced, row-major
    // LDS store).  V chunks: the 64 lanes of a wave hold 64 consecutive keys of
    // one column chunk, so the transposed LDS stores of a wave hit consecutive
    // addresses.
    uint4 rk[PER_T], rv[PER_T];
    auto k_chunk = [&](int u, int &key, int &dc) {
        const int ci = tid + u * 256;
        key = ci / (HD / CH);
        dc = (ci % (HD / CH)) * CH;
    };
    auto v_chunk = [&](int u, int &key, int &dc) {
        const int ci = tid + u * 256;
        key = ci % KT;
        dc = (ci / KT) * CH;
    };
    auto gload = [&](int i) {
        const bool sfx = i >= n_pre;
        const int k0 = sfx ? blk.sfx_lo + (i - n_pre) * KT : blk.key0 + i * KT;
        const int kl = sfx ? blk.sfx_hi : kmax;
        const T *Ksrc = sfx ? Kb : Kg, *Vsrc = sfx ? Vb : Vg;
#pragma unroll
        for (int u = 0; u < PER_T; ++u) {
            int key, dc;
            k_chunk(u, key, dc);
            rk[u] = k0 + key < kl ? *reinterpret_cast<const uint4 *>(Ksrc + (size_t)(k0 + key) * HD + dc)
                                  : make_uint4(0, 0, 0, 0);
            v_chunk(u, key, dc);
            rv[u] = k0 + key < kl ? *reinterpret_cast<const uint4 *>(Vsrc + (size_t)(k0 + key) * HD + dc)
                                  : make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](T *Ks, T *Vt) {
#pragma unroll
        for (int u = 0; u < PER_T; ++u) {
            int key, dc;
            k_chunk(u, key, dc);
            *reinterpret_cast<uint4 *>(Ks + key * LDKS + dc) = rk[u];
            v_chunk(u, key, dc);
            const T *ve = reinterpret_cast<const T *>(&rv[u]);
#pragma unroll
            for (int e = 0; e < CH; ++e) Vt[(dc + e) * LDV + key] = ve[e];
        }
    };

    float m_run = -INFINITY, l_run = 0.f;  // stats of query row lr (replicated over lg)
    f32x4 o[CF];
#pragma unroll
    for (int j = 0; j < CF; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (n_tiles > 0) {
        gload(0);
        lstore(Ks0, Vt0);
    }
    __syncthreads();
    for (int i = 0; i < n_tiles; ++i) {
        T *Ks = (i & 1) ? Ks1 : Ks0, *Vt = (i & 1) ? Vt1 : Vt0;
        if (i + 1 < n_tiles) gload(i + 1);
        const bool sfx = i >= n_pre;
        const int k0 = sfx ? blk.sfx_lo + (i - n_pre) * KT : blk.key0 + i * KT;

        // S^T tile: sc[kf][r] = score(query lr, key k0 + kf*16 + 4*lg + r).  Every
        // K fragment of the tile is read before the first multiply, and the
        // multiplies interleave four independent accumulators.
        f32x4 sc[KT / 16];
        {
            Frag<T> kfr[KT / 16][HS];
#pragma unroll
            for (int kf = 0; kf < KT / 16; ++kf)
#pragma unroll
                for (int st = 0; st < HS; ++st) ld8(kfr[kf][st], Ks + (kf * 16 + lr) * LDKS + st * 32 + lg * 8);
            __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the multiplies
#pragma unroll
            for (int kf = 0; kf < KT / 16; ++kf) sc[kf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < HS; ++st)
#pragma unroll
                for (int kf = 0; kf < KT / 16; ++kf) mma(sc[kf], kfr[kf][st], qf[st]);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kf = 0; kf < KT / 16; ++kf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + kf * 16 + lg * 4 + r;
                bool see;
                if (!sfx) see = key < kend_row;
                else see = row_ok && key < blk.sfx_hi && row_vis_sees(vis, c, key);
                const float v = see ? sc[kf][r] * qscale : -INFINITY;
                sc[kf][r] = v;
                mx = fmaxf(mx, v);
            }
        mx = rows_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
        float psum = 0.f;
        float pr[KT / 16][4];
#pragma unroll
        for (int kf = 0; kf < KT / 16; ++kf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pr[kf][r] = __builtin_amdgcn_exp2f(sc[kf][r] - m_ref);
                psum += pr[kf][r];
            }
        // this lane's share of the row sum; the four shares are added at the end
        l_run = l_run * alpha + psum;
        m_run = m_new;

        // rescale O: its rows are queries 4*lg + r, whose alpha sits in lane 4*lg + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float a = __shfl(alpha, lg * 4 + r);
#pragma unroll
            for (int j = 0; j < CF; ++j) o[j][r] *= a;
        }
        // O += P V over two 32-key steps; A = P (row lr, keys {4lg..4lg+3} and {16+4lg..}), B = V.
        // All V fragments are read first.
        {
            Frag<T> vfr[KT / 32][CF];
#pragma unroll
            for (int st = 0; st < KT / 32; ++st)
#pragma unroll
                for (int j = 0; j < CF; ++j) {
                    const T *vrow = Vt + (j * 16 + lr) * LDV + st * 32 + lg * 4;
                    ld4x2(vfr[st][j], vrow, vrow + 16);
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int st = 0; st < KT / 32; ++st) {
                float pv[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pv[r] = pr[2 * st][r];
                    pv[4 + r] = pr[2 * st + 1][r];
                }
                Frag<T> pa;
                from8(pa, pv);
#pragma unroll
                for (int j = 0; j < CF; ++j) mma(o[j], pa, vfr[st][j]);
            }
        }
        // tile i+1 goes into the other buffer, last read during iteration i-1
        if (i + 1 < n_tiles) lstore((i & 1) ? Ks0 : Ks1, (i & 1) ? Vt0 : Vt1);
        __syncthreads();
    }

    attn_write<T, HD>(c, blk, o, m_run, rows_sum(l_run), w, lr, lg);
}

// ---------------------------------------------------------------------------
// Attention for 16-bit types.  Same rows, keys, masks and outputs as k_attn,
// but the operands never pass through registers on their way to LDS: the
// 64 query rows and every (K, V) tile of 64 keys are copied by LDS-DMA
// (global_load_lds_dwordx4), the key tiles through an S-stage ring so that
// S-1 tiles are in flight while the matrix cores work on the current one.
// A DMA instruction writes 1 KB linearly, so the LDS tiles are unpadded and
// bank conflicts are avoided by permuting the 16-byte chunks of each row:
// K and Q rows keep chunk c at c ^ (row % CPR), which spreads the 16 rows of
// an MFMA fragment read over all banks; V rows keep chunk c at
// c ^ (2*row % CPR), which does the same for the 4 rows of gfx950's LDS
// transpose read (ds_read_b64_tr_b16) that delivers V's MFMA fragments.
// ---------------------------------------------------------------------------
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
// Four 16-bit values by the LDS transpose read: within each 16-lane row of
// the wave, lane j names 8 bytes (4 values); lane i receives value i % 4 of
// the groups named by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12.
__device__ __forceinline__ short4_t lds_tr4(const char *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4_t *)(__attribute__((address_space(3))) const char *)p);
}

// A row's running maximum is raised (and its partial sums rescaled) only when
// a tile's maximum exceeds it by more than this many powers of two; between
// raises the exponentials stay below 2^RESCALE_LOG2, which bf16 holds at full
// relative precision, and the normalised result is the same softmax.
constexpr float RESCALE_LOG2 = 8.0f;
// Key-tile ring depth.  Each tile's work is bound by latency (about 1 us per
// 64-key tile for a 4-wave block), so two stages suffice, and the smaller
// ring (80 KB of LDS at head_dim 128) lets two blocks share a CU: the
// 64 x 1,024-token batched prefill's attention takes 0.57 ms per layer instead
// of 0.87 ms with three stages; a 252-block launch is unchanged.
#ifndef ATT_RING_STAGES
#define ATT_RING_STAGES 2
#endif

template <int HD> struct RingLds {
    static constexpr int KT = 64, RB = HD * 2, CPR = RB / 16, TILE = KT * RB;
    static constexpr int Q_BYTES = TILE;  // 64 query rows
    // H key rings (one per half of the workgroup) behind the query rows.
    // RW = 2 (128 query rows): the rows wait in the ring's second slot,
    // which they fill exactly, until every wave holds its own in registers.
    static int bytes(int S, int H = 1, int RW = 1) { return (RW == 2 ? 0 : Q_BYTES) + H * S * 2 * TILE; }
};

// H = 2: a workgroup of 8 waves, whose halves (waves 0-3 and 4-7) walk the
// first and the second half of the block's key tiles, each through its own
// ring, for the same 64 query rows; at the end the second half's (max, sum,
// O) go through LDS to the first, which merges them and writes the rows.
// Each key chain is half as long, two waves share each SIMD, and no merge
// kernel runs.  Used for launches of at most 256 blocks, where each block
// has a compute unit to itself anyway (the two rings fill 144 KB of LDS).
//
// RW = 2: 128 query rows, two 16-row groups per wave (rows 32 w .. 32 w +
// 31).  Every K and V fragment a wave reads from LDS feeds both groups'
// matrix instructions, which halves the LDS bytes per flop: with one group
// per wave, the K and V reads of a tile take twice the LDS cycles of its
// matrix work.  Causal prefix blocks only (no branch keys); the 64 KB ring
// keeps two blocks on a compute unit.
template <int HD, int S, int H = 1, int RW = 1>
__global__ __launch_bounds__(256 * H) void k_attn_ring(AttnCall c) {
    using T = bf16_t;
    using L = RingLds<HD>;
    constexpr int KT = L::KT, RB = L::RB, CPR = L::CPR, TILE = L::TILE, STAGE = 2 * TILE;
    constexpr int INS = TILE / (4 * 1024);  // DMA instructions per wave per tile
    constexpr int LPS = 2 * INS;            // per (K, V) stage
    constexpr int HS = HD / 32, CF = HD / 16;
    static_assert(INS >= 1 && INS * 4 * 1024 == TILE, "tile / DMA mapping");
    static_assert(S >= 2 && (S - 1) * LPS + INS < 64, "vmcnt range");
    static_assert(H == 1 || (H == 2 && S == 2), "two halves with two-stage rings");
    static_assert(RW == 1 || (RW == 2 && H == 1 && S == 2), "128-row blocks: one 4-wave ring of two stages");
    extern __shared__ __attribute__((aligned(16))) char attn_lds[];
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)attn_lds;
    constexpr int Q_OFF = RW == 2 ? STAGE : 0;  // the query rows: ring slot 1 (RW = 2) or ahead of the ring
    const char *Qs = attn_lds + Q_OFF;

    const AttnBlock blk = c.blocks[blockIdx.x];
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int half = (tid >> 6) / 4, w = (tid >> 6) % 4;  // w: this wave's query rows 16 RW w .. 16 RW (w + 1) - 1
    const uint32_t ring_off = (uint32_t)((RW == 2 ? 0 : L::Q_BYTES) + half * S * STAGE);  // this half's key ring
    const uint32_t ring_base = lds_base + ring_off;
    const int Hq = c.n_heads, Hkv = c.n_kv_heads, grp = Hq / Hkv;
    const int P = c.req_stride[blk.req];  // slab stride (the buffer's token capacity)
    const char *kvbase = reinterpret_cast<const char *>(c.req_kv[blk.req]);
    const char *Kg = kvbase + ((size_t)c.layer * 2 * Hkv + blk.g) * (size_t)P * RB;
    const char *Vg = kvbase + ((size_t)c.layer * 2 * Hkv + Hkv + blk.g) * (size_t)P * RB;
    const char *Kb = reinterpret_cast<const char *>(c.kb) + (size_t)blk.g * c.cap * RB;
    const char *Vb = reinterpret_cast<const char *>(c.vb) + (size_t)blk.g * c.cap * RB;
    const float qscale = LOG2E / sqrtf((float)HD);

    // this lane's query rows (B operand of S^T), one per 16-row group, and their tokens
    bool row_ok[RW];
    int tq[RW], kend_row[RW];
#pragma unroll
    for (int rb = 0; rb < RW; ++rb) {
        const int lrow = (w * RW + rb) * 16 + lr;
        row_ok[rb] = lrow < blk.nrows;
        tq[rb] = (row_ok[rb] ? blk.row0 + lrow : blk.row0) / grp;
        kend_row[rb] = blk.causal ? min(blk.qoff + tq[rb] + 1, blk.key1) : blk.key1;
    }
    // keys below kend_lo are visible to every row of the block (its first row's bound)
    const int kend_lo = blk.causal ? min(blk.qoff + blk.row0 / grp + 1, blk.key1) : blk.key1;
    int kmax = blk.key1;
    if (blk.causal) {
        const int last = blk.qoff + (blk.row0 + blk.nrows - 1) / grp + 1;
        kmax = last < kmax ? last : kmax;
    }
    const int n_pre = kmax > blk.key0 ? (kmax - blk.key0 + KT - 1) / KT : 0;
    // branch keys: 64-row blocks only (the host never gives them to 128-row blocks)
    const int n_sfx = (RW == 1 && blk.sfx_hi > blk.sfx_lo) ? (blk.sfx_hi - blk.sfx_lo + KT - 1) / KT : 0;
    const int n_tiles = n_pre + n_sfx;
    // this half's tiles: global indices [t_base, t_base + t_cnt); both halves
    // run n_iter loop steps, so they meet every barrier the same number of times
    const int n_iter = H == 1 ? n_tiles : (n_tiles + 1) / 2;
    const int t_base = half * n_iter, t_cnt = half == 0 ? n_iter : n_tiles - n_iter;
    RowVis vis{};
    if (n_sfx > 0) {
        row_vis_init(vis, c, tq[0] - c.branch0);
        vm_wait<0>();  // its loads must not sit in the counter behind the DMA below
    }

    // DMA slots of this lane: 16-byte unit p = (i*4 + w)*64 + lane of a tile,
    // row p / CPR, physical chunk p % CPR, logical chunk per the row permutation
    int drow[INS], dck[INS], dcv[INS];
#pragma unroll
    for (int i = 0; i < INS; ++i) {
        const int p = (i * 4 + w) * 64 + lane, pc = p % CPR;
        drow[i] = p / CPR;
        dck[i] = pc ^ (drow[i] & (CPR - 1));
        dcv[i] = pc ^ ((2 * drow[i]) & (CPR - 1));
    }
    // query rows: (token, head) pairs of this block; rows past nrows re-read row0
    // (loaded by the first half; the second reads them after the first barrier).
    // Rows 64 h2 .. 64 h2 + 63 take the layout of one key tile, TILE bytes on.
    if (half == 0) {
        const char *Q = reinterpret_cast<const char *>(c.q);
#pragma unroll
        for (int h2 = 0; h2 < RW; ++h2)
#pragma unroll
            for (int i = 0; i < INS; ++i) {
                const int qi = h2 * 64 + drow[i];
                const int qr = qi < blk.nrows ? blk.row0 + qi : blk.row0;
                const size_t qrow = (size_t)(qr / grp) * Hq + blk.g * grp + qr % grp;
                dma16(Q + qrow * RB + dck[i] * 16, lds_base + (uint32_t)(Q_OFF + h2 * TILE + (i * 4 + w) * 1024));
            }
    }
    auto issue = [&](int i, int it) {  // tile i into ring slot it % S
        const bool sfx = i >= n_pre;
        const int k0 = sfx ? blk.sfx_lo + (i - n_pre) * KT : blk.key0 + i * KT;
        const int kl = sfx ? blk.sfx_hi : kmax;
        const char *Ksrc = sfx ? Kb : Kg, *Vsrc = sfx ? Vb : Vg;
        const uint32_t sb = ring_base + (uint32_t)((it % S) * STAGE);
#pragma unroll
        for (int u = 0; u < INS; ++u) {
            const size_t key = (size_t)min(k0 + drow[u], kl - 1);  // keys past the range: a valid key, masked below
            dma16(Ksrc + key * RB + dck[u] * 16, sb + (uint32_t)((u * 4 + w) * 1024));
            dma16(Vsrc + key * RB + dcv[u] * 16, sb + (uint32_t)(TILE + (u * 4 + w) * 1024));
        }
    };
#pragma unroll
    for (int s = 0; s + 1 < S; ++s)
        if (s < t_cnt) issue(t_base + s, s);

    // per 16-row group rb: reference max of query row lr (replicated over lg); this lane's share of the sum
    float m_run[RW], l_run[RW];
    f32x4 o[RW][CF];
    Frag<T> qf[RW][HS];
#pragma unroll
    for (int rb = 0; rb < RW; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
#pragma unroll
        for (int j = 0; j < CF; ++j) o[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    auto frag16 = [&](const char *tile, int row, int lc) {  // 16 bytes: logical chunk lc of a K or Q row
        Frag<T> f;
        f.v = *reinterpret_cast<const bf16x8_t *>(tile + row * RB + ((lc ^ (row & (CPR - 1))) * 16));
        return f;
    };

    // One key tile from ring slot i % S: prefix keys (SFX false: visible below
    // kend_row) or branch keys (SFX true: the row's scaffold and trie ancestors).
    auto tile = [&](auto SFXC, int i, int it) {  // tile i from ring slot it % S
        constexpr bool SFX = decltype(SFXC)::value;
        const char *Kt = attn_lds + ring_off + (it % S) * STAGE, *Vt = Kt + TILE;
        const int k0 = SFX ? blk.sfx_lo + (i - n_pre) * KT : blk.key0 + i * KT;

        // S^T tile: sc[rb][kf][r] = score(query 16 rb + lr, key k0 + kf*16 + 4*lg + r)
        f32x4 sc[RW][KT / 16];
        {
            Frag<T> kfr[KT / 16][HS];
#pragma unroll
            for (int kf = 0; kf < KT / 16; ++kf)
#pragma unroll
                for (int st = 0; st < HS; ++st) kfr[kf][st] = frag16(Kt, kf * 16 + lr, st * 4 + lg);
            __builtin_amdgcn_sched_barrier(0);  // every read ahead of the multiplies
#pragma unroll
            for (int rb = 0; rb < RW; ++rb)
#pragma unroll
                for (int kf = 0; kf < KT / 16; ++kf) sc[rb][kf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < HS; ++st)
#pragma unroll
                for (int kf = 0; kf < KT / 16; ++kf)
#pragma unroll
                    for (int rb = 0; rb < RW; ++rb) mma(sc[rb][kf], kfr[kf][st], qf[rb][st]);
        }
        float pr[RW][KT / 16][4];
#pragma unroll
        for (int rb = 0; rb < RW; ++rb) {
            // Row maximum of the raw scores (masked keys set to -inf), then scaled:
            // the scale is positive, so this equals the maximum of the scaled
            // scores.  A prefix tile below every row's causal bound needs no mask.
            float mx = -INFINITY;
            if (!SFX && k0 + KT <= kend_lo) {
#pragma unroll
                for (int kf = 0; kf < KT / 16; ++kf)
#pragma unroll
                    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[rb][kf][r]);
            } else {
#pragma unroll
                for (int kf = 0; kf < KT / 16; ++kf)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = k0 + kf * 16 + lg * 4 + r;
                        bool see;
                        if constexpr (SFX) see = row_ok[rb] && key < blk.sfx_hi && row_vis_sees(vis, c, key);
                        else see = key < kend_row[rb];
                        const float v = see ? sc[rb][kf][r] : -INFINITY;
                        sc[rb][kf][r] = v;
                        mx = fmaxf(mx, v);
                    }
            }
            mx = rows_max(mx) * qscale;
            if (__any(mx > m_run[rb] + RESCALE_LOG2)) {
                const float m_new = fmaxf(m_run[rb], mx);
                const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - (m_new == -INFINITY ? 0.f : m_new));
                l_run[rb] *= alpha;
                m_run[rb] = m_new;
                // o holds this lane's own query row lr (columns 16 j + 4 lg + r)
#pragma unroll
                for (int j = 0; j < CF; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[rb][j][r] *= alpha;
            }
            const float m_neg = m_run[rb] == -INFINITY ? 0.f : -m_run[rb];
            float psum = 0.f;
#pragma unroll
            for (int kf = 0; kf < KT / 16; ++kf)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pr[rb][kf][r] = __builtin_amdgcn_exp2f(fmaf(sc[rb][kf][r], qscale, m_neg));
                    psum += pr[rb][kf][r];
                }
            l_run[rb] += psum;
        }

        // O += P V over two 32-key steps; A = P (row lr, keys {4lg..4lg+3} and
        // {16+4lg..16+4lg+3}), B = V with the same key order: lane (lr, lg)
        // names key rows 32st + 4lg + lr/4 (and +16), columns 16j + 4(lr%4)..+3.
        Frag<T> vfr[KT / 32][CF];
#pragma unroll
        for (int st = 0; st < KT / 32; ++st)
#pragma unroll
            for (int j = 0; j < CF; ++j) {
                const int row = st * 32 + lg * 4 + (lr >> 2);
                const int pc = (2 * j + ((lr & 3) >> 1)) ^ ((2 * row) & (CPR - 1));  // same for row + 16
                const char *v0 = Vt + row * RB + pc * 16 + 8 * (lr & 1);
                const short4_t lo = lds_tr4(v0), hi = lds_tr4(v0 + 16 * RB);
                const short8_t both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                vfr[st][j].v = __builtin_bit_cast(bf16x8_t, both);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < KT / 32; ++st)
#pragma unroll
            for (int rb = 0; rb < RW; ++rb) {
                float pv[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pv[r] = pr[rb][2 * st][r];
                    pv[4 + r] = pr[rb][2 * st + 1][r];
                }
                Frag<T> pa;
                from8(pa, pv);
#pragma unroll
                for (int j = 0; j < CF; ++j) mma(o[rb][j], vfr[st][j], pa);  // V first: o[j] is O^T's layout
            }
    };

    for (int it = 0; it < n_iter; ++it) {
        // this step's tile (and the query rows) landed: later tiles issued so far may stay in flight
        vm_wait_ahead<LPS, S - 2>(max(0, min(S - 2, t_cnt - 1 - it)));
        barrier_keep_loads();
        if (it == 0) {
#pragma unroll
            for (int rb = 0; rb < RW; ++rb)
#pragma unroll
                for (int st = 0; st < HS; ++st) qf[rb][st] = frag16(Qs, (w * RW + rb) * 16 + lr, st * 4 + lg);
            if constexpr (RW == 2) {
                // the query rows sit in slot 1, which the next issue refills
                lds_reads_done();
                barrier_keep_loads();
            }
        }
        // slot (it - 1) % S was read by every wave of this half before the barrier
        if (it + S - 1 < t_cnt) issue(t_base + it + S - 1, it + S - 1);
        if (it < t_cnt) {
            const int i = t_base + it;
            if (i < n_pre) tile(std::false_type{}, i, it);
            else if constexpr (RW == 1) tile(std::true_type{}, i, it);
        }
        lds_reads_done();
    }
    if constexpr (H == 2) {
        // the second half hands its (O, max, sum share) per lane to the
        // same lane of the first half's wave with the same query rows,
        // through its own ring (free once every wave has passed this barrier)
        constexpr int NV = 4 * CF + 2;
        float *xs = reinterpret_cast<float *>(attn_lds + L::Q_BYTES + S * STAGE) + w * NV * 64 + lane;
        static_assert(4 * NV * 64 * 4 <= S * STAGE, "hand-over area");
        __syncthreads();
        if (half == 1) {
#pragma unroll
            for (int j = 0; j < CF; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) xs[(j * 4 + r) * 64] = o[0][j][r];
            xs[4 * CF * 64] = m_run[0];
            xs[(4 * CF + 1) * 64] = l_run[0];
        }
        __syncthreads();
        if (half == 1) return;
        // merge: the common reference is the larger maximum (log2 units)
        const float m1 = xs[4 * CF * 64], l1 = xs[(4 * CF + 1) * 64];
        const float mm = fmaxf(m_run[0], m1);
        const float a0 = m_run[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[0] - mm);
        const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
        l_run[0] = l_run[0] * a0 + l1 * a1;
        m_run[0] = mm;
#pragma unroll
        for (int j = 0; j < CF; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[0][j][r] = o[0][j][r] * a0 + xs[(j * 4 + r) * 64] * a1;
    }
#pragma unroll
    for (int rb = 0; rb < RW; ++rb)
        attn_write_rows<T, HD>(c, blk, o[rb], m_run[rb], rows_sum(l_run[rb]), w * RW + rb, lr, lg);
}


template <int HD, int S, int H, int RW = 1> static void launch_attn_ring_h(const AttnCall &c, hipStream_t st) {
    const int shmem = RingLds<HD>::bytes(S, H, RW);
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(k_attn_ring<HD, S, H, RW>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, shmem);
        attr_set = true;
    }
    hipLaunchKernelGGL((k_attn_ring<HD, S, H, RW>), dim3(c.n_blocks), dim3(256 * H), shmem, st, c);
}
// Launches of at most one block per compute unit split each block's key
// chain over two halves of one workgroup; larger ones keep 4-wave blocks,
// two of which share a compute unit, unless the host asks for two chains
// (a launch bound by its longest chains).
template <int HD, int S> static void launch_attn_ring(const AttnCall &c, hipStream_t st) {
    if constexpr (S == 2) {
        if (c.wide) {
            launch_attn_ring_h<HD, S, 1, 2>(c, st);
            return;
        }
        if (c.n_blocks <= ATT_HALVES_MAX_BLOCKS || c.halves) {
            launch_attn_ring_h<HD, S, 2>(c, st);
            return;
        }
    }
    launch_attn_ring_h<HD, S, 1>(c, st);
}

template <typename T, int HD> static int attn_lds_bytes() {
    constexpr int KPAD = 16 / sizeof(T);
    return 2 * (64 * (HD + KPAD) + HD * (64 + KPAD)) * (int)sizeof(T);
}

template <typename T, int HD> static void launch_attn(const AttnCall &c, hipStream_t st) {
    const int shmem = attn_lds_bytes<T, HD>();
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(k_attn<T, HD>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, shmem);
        attr_set = true;
    }
    hipLaunchKernelGGL((k_attn<T, HD>), dim3(c.n_blocks), dim3(256), shmem, st, c);
}

template <typename T> static bool attention_t(const AttnCall &c, hipStream_t st) {
    if (c.n_blocks <= 0) return true;
    if (c.wide && (sizeof(T) != 2 || ATT_RING_STAGES != 2)) return false;  // 128-row blocks: the two-stage bf16 ring only
    if constexpr (sizeof(T) == 2) {
        switch (c.hd) {
            case 32: launch_attn_ring<32, ATT_RING_STAGES>(c, st); return true;
            case 64: launch_attn_ring<64, ATT_RING_STAGES>(c, st); return true;
            case 128: launch_attn_ring<128, ATT_RING_STAGES>(c, st); return true;
        }
    } else {
        switch (c.hd) {
            case 32: launch_attn<T, 32>(c, st); return true;
            case 64: launch_attn<T, 64>(c, st); return true;
        }
    }
    return false;
}
bool attention(const AttnCall &c, hipStream_t st) {
    return c.dt == PCD_DT_F32 ? attention_t<float>(c, st) : attention_t<bf16_t>(c, st);
}

// Merge the split partials of each (token, head) of the requests that used
// more than one split: m = max, l = sum l_s 2^(m_s - m), O = sum O_s 2^(m_s - m).
// Every split's loads go out before the first is used (one memory round trip
// per (token, head) rather than one per split); SMAX bounds the split count.
template <typename T, int HD, int SMAX>
__global__ __launch_bounds__(256) void k_attn_merge(TailCall c) {
    constexpr int PL = (HD + 63) / 64;
    const int lane = threadIdx.x & 63;
    const int id = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int Hq = c.n_heads;
    if (id >= (c.n_tokens - c.tok0) * Hq) return;
    const int t = c.tok0 + id / Hq, h = id % Hq;
    const int ns = c.tok_splits[t];
    if (ns <= 1) return;  // written directly by the attention kernel
    float2 ml[SMAX];
    float po[SMAX][PL];
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
        if (s >= ns) break;
        const size_t pi = ((size_t)s * c.n_tokens + t) * Hq + h;
        ml[s] = c.part_ml[pi];
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const int d = lane + 64 * i;
            po[s][i] = d < HD ? c.part_o[pi * HD + d] : 0.f;
        }
    }
    float m = -INFINITY, l = 0.f, o[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) o[i] = 0.f;
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
        if (s >= ns) break;
        const float mn = fmaxf(m, ml[s].x);
        const float a = __builtin_amdgcn_exp2f(m - mn), b = __builtin_amdgcn_exp2f(ml[s].x - mn);
#pragma unroll
        for (int i = 0; i < PL; ++i) o[i] = o[i] * a + po[s][i] * b;
        l = l * a + ml[s].y * b;
        m = mn;
    }
    T *out = reinterpret_cast<T *>(c.out) + ((size_t)t * Hq + h) * HD;
    const float inv = 1.0f / l;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int d = lane + 64 * i;
        if (d < HD) out[d] = from_f<T>(o[i] * inv);
    }
}

template <typename T> static void merge_t(const TailCall &c, hipStream_t st) {
    const int waves = (c.n_tokens - c.tok0) * c.n_heads;
    if (waves <= 0) return;
    const dim3 grid((waves + 3) / 4);
    switch (c.hd) {
        case 32: hipLaunchKernelGGL((k_attn_merge<T, 32, ATT_MAX_SPLITS>), grid, dim3(256), 0, st, c); break;
        case 64: hipLaunchKernelGGL((k_attn_merge<T, 64, ATT_MAX_SPLITS>), grid, dim3(256), 0, st, c); break;
        case 128: hipLaunchKernelGGL((k_attn_merge<T, 128, ATT_MAX_SPLITS>), grid, dim3(256), 0, st, c); break;
    }
}
void attention_merge(const TailCall &c, hipStream_t st) {
    if (c.dt == PCD_DT_F32) merge_t<float>(c, st);
    else merge_t<bf16_t>(c, st);
}

// ---------------------------------------------------------------------------
// readout statistics and the per-field combine
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_readout_lse(const float2 *part, int32_t n_tiles, int32_t R, float *lse) {
    __shared__ float red[4];
    const int r = blockIdx.x;
    float mx = -INFINITY;
    for (int i = threadIdx.x; i < n_tiles; i += 256) mx = fmaxf(mx, part[(size_t)i * R + r].x);
    mx = wave_max(mx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float s = 0.f;
    for (int i = threadIdx.x; i < n_tiles; i += 256) {
        const float2 p = part[(size_t)i * R + r];
        s += p.y * __expf(p.x - mx);
    }
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) lse[r] = mx + logf(red[0] + red[1] + red[2] + red[3]);
}

// Gather of rows for the last layer of a pass: block i < n copies row
// rows[i] of a, block n + i that of b, in 16-byte units.
__global__ __launch_bounds__(256) void k_gather_rows2(const uint4 *src_a, int32_t vec_a, uint4 *dst_a,
                                                      const uint4 *src_b, int32_t vec_b, uint4 *dst_b,
                                                      const int32_t *rows, int32_t n) {
    const bool second = (int)blockIdx.x >= n;
    const int i = second ? blockIdx.x - n : blockIdx.x;
    const int vec = second ? vec_b : vec_a;
    const uint4 *src = (second ? src_b : src_a) + (size_t)rows[i] * vec;
    uint4 *dst = (second ? dst_b : dst_a) + (size_t)i * vec;
    for (int j = threadIdx.x; j < vec; j += 256) dst[j] = src[j];
}

void gather_rows2(const void *src_a, size_t bytes_a, void *dst_a, const void *src_b, size_t bytes_b, void *dst_b,
                  const int32_t *rows, int32_t n, hipStream_t st) {
    if (n <= 0) return;
    hipLaunchKernelGGL(k_gather_rows2, dim3(2 * n), dim3(256), 0, st, reinterpret_cast<const uint4 *>(src_a),
                       (int32_t)(bytes_a / 16), reinterpret_cast<uint4 *>(dst_a), reinterpret_cast<const uint4 *>(src_b),
                       (int32_t)(bytes_b / 16), reinterpret_cast<uint4 *>(dst_b), rows, n);
}

// The same arithmetic in the same order for up to 256 * KMAX tiles, with each
// thread's partials loaded once into registers (one memory round trip).
constexpr int LSE_KMAX = 8;
__global__ __launch_bounds__(256) void k_readout_lse_reg(const float2 *part, int32_t n_tiles, int32_t R, float *lse) {
    __shared__ float red[4];
    const int r = blockIdx.x, tid = threadIdx.x;
    float2 p[LSE_KMAX];
#pragma unroll
    for (int k = 0; k < LSE_KMAX; ++k) {
        const int i = tid + 256 * k;
        p[k] = i < n_tiles ? part[(size_t)i * R + r] : make_float2(-INFINITY, 0.f);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < LSE_KMAX; ++k) mx = fmaxf(mx, p[k].x);
    mx = wave_max(mx);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < LSE_KMAX; ++k)
        if (tid + 256 * k < n_tiles) s += p[k].y * __expf(p[k].x - mx);
    s = wave_sum(s);
    if ((tid & 63) == 0) red[tid >> 6] = s;
    __syncthreads();
    if (tid == 0) lse[r] = mx + logf(red[0] + red[1] + red[2] + red[3]);
}

void readout_lse(const float2 *part, int32_t n_tiles, int32_t R, float *lse, hipStream_t st) {
    if (R <= 0) return;
    if (n_tiles <= 256 * LSE_KMAX)
        hipLaunchKernelGGL(k_readout_lse_reg, dim3(R), dim3(256), 0, st, part, n_tiles, R, lse);
    else hipLaunchKernelGGL(k_readout_lse, dim3(R), dim3(256), 0, st, part, n_tiles, R, lse);
}

// One thread per field.  A spelling's score sums the log-probabilities of the
// edges on its path: z - lse (full vocabulary), or in SCORE_LEVEL z minus
// the log-sum-exp of its readout's gathered child logits; SCORE_MEAN
// divides the sum by the path length.  A label's score is the log-sum-exp of
// its spellings' scores.  The scores are written to c.logscore first and read
// back from there (same thread).
// One wave per field: lane l scores candidates c0 + l, c0 + l + 64, ...
// (each with its own spellings and paths), then the wave reduces the
// maximum (ties to the lowest candidate index), the runner-up, the softmax
// denominator and the mass.  The 255-option ID field is 4 candidates per
// lane instead of a serial loop of 255.
__global__ __launch_bounds__(64) void k_combine(CombineCall c) {
    const int f = blockIdx.x, lane = threadIdx.x;
    const int c0 = c.f_cand_off[f], c1 = c.f_cand_off[f + 1];
    const int mode = c.f_mode[f];
    auto norm = [&](int r) {
        if (mode != SCORE_LEVEL) return c.lse[r];
        float mx = -INFINITY;
        for (int gi = c.g_off[r]; gi < c.g_off[r + 1]; ++gi) mx = fmaxf(mx, c.z[gi]);
        float sum = 0.f;
        for (int gi = c.g_off[r]; gi < c.g_off[r + 1]; ++gi) sum += __expf(c.z[gi] - mx);
        return mx + __logf(sum);
    };
    auto spelling = [&](int sp) {
        float s = 0.f;
        const int i0 = c.s_path_off[sp], i1 = c.s_path_off[sp + 1];
        for (int i = i0; i < i1; ++i) {
            const int gi = c.s_path[i];
            s += c.z[gi] - norm(c.g_ro[gi]);
        }
        return mode == SCORE_MEAN ? s / (float)(i1 - i0) : s;
    };
    // this lane's candidates: their scores, the lane's best (first on ties)
    float best = -INFINITY;
    int arg = c1;  // past the field: no candidate on this lane
    for (int k = c0 + lane; k < c1; k += 64) {
        const int s0 = c.c_spell_off[k], s1 = c.c_spell_off[k + 1];
        float s = spelling(s0);
        if (s1 - s0 > 1) {
            float mx = s;
            for (int sp = s0 + 1; sp < s1; ++sp) mx = fmaxf(mx, spelling(sp));
            float sum = 0.f;
            for (int sp = s0; sp < s1; ++sp) sum += __expf(spelling(sp) - mx);
            s = mx + __logf(sum);
        }
        c.logscore[k] = s;
        if (s > best) {
            best = s;
            arg = k;
        }
    }
    // wave maximum; equal values go to the lower candidate index
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ob = __shfl_xor(best, o);
        const int oa = __shfl_xor(arg, o);
        if (ob > best || (ob == best && oa < arg)) {
            best = ob;
            arg = oa;
        }
    }
    // the runner-up: the largest score of every other candidate (equal to the
    // best when two candidates tie); the lane's own writes are visible to it
    float second = -INFINITY;
    for (int k = c0 + lane; k < c1; k += 64)
        if (k != arg) second = fmaxf(second, c.logscore[k]);
    second = wave_max(second);
    const float invT = 1.0f / c.temperature;
    float den = 0.f;
    for (int k = c0 + lane; k < c1; k += 64) den += __expf((c.logscore[k] - best) * invT);
    den = wave_sum(den);
    for (int k = c0 + lane; k < c1; k += 64) c.prob[k] = __expf((c.logscore[k] - best) * invT) / den;
    const int root = c.f_ro_root[f];
    float mass = 0.f;
    for (int gi = c.g_off[root] + lane; gi < c.g_off[root + 1]; gi += 64) mass += __expf(c.z[gi] - c.lse[root]);
    mass = wave_sum(mass);
    if (lane == 0) {
        c.mass[f] = mass;
        c.margin[f] = best - second;
        c.argmax[f] = arg - c0;
    }
}

void combine(const CombineCall &c, hipStream_t st) {
    if (c.n_fields <= 0) return;
    hipLaunchKernelGGL(k_combine, dim3(c.n_fields), dim3(64), 0, st, c);
}

}  // namespace pcd
