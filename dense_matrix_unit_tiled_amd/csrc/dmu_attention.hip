// Fused attention forward on the matrix cores: O = softmax(scale Q K^T) V.
//
// The pages move the two products of a FlashAttention kernel onto the matrix
// units and keep P = softmax(S) in registers between them (layout-experiment
// post, sections 1-2; "Tensor Cores, CUTLASS and CuTe", part 3 section 2: the
// accumulator of S = Q K^T is reused as an operand of O = P V, and each row's
// max and sum are taken across the lanes that share the row).  This is that
// computation for gfx950, one pass over the keys with the online softmax:
//
//   workgroup   8 wavefronts, 256 query rows of one batch slice (32 per
//               wavefront: two 16-row tiles), walking the keys in blocks of 64;
//               workgroups renumbered so that one batch slice's query blocks
//               share an XCD (and its L2 copy of K and V).
//   K, V        64-key blocks through the GEMM kernel's register-staged LDS
//               path, in two rings of two buffers: K (K-contiguous layout, two
//               64 x 64 halves of the head dimension) one block ahead of V
//               (transposed layout).  One barrier per block.
//   S = Q K^T   MFMA(srcA = K fragment, srcB = Q fragment) on 16 x 16 tiles: lane
//               l owns S[q = l % 16][key = 16 t + 4 (l / 16) + r] of key tile t.
//               Q's fragments stay in registers for the whole pass.
//   pipeline    step j computes the scores of block j+1 while block j's
//               softmax runs (independent work for the matrix core and the
//               VALU in one region) and takes block j+1's row maxima, then
//               O += P V for block j.
//   softmax     in base 2 with c = scale log2(e) >= 0 (a negative scale negates
//               Q instead): per row a running maximum m of c s (across the four
//               lanes that share the row), raised only when a block's maximum
//               passes it by more than 8 -- decided at the start of the block's
//               step from each lane's own maximum, where the maximum across the
//               lanes and the correction 2^(m_old - m_new) of O and l are a
//               rarely taken branch -- then p = 2^(c s - m) <= 2^8 (one FMA and
//               the hardware exp2) and the running sum l (kept per lane, added
//               up at the end).  Only the last block can hold keys past seq_k;
//               they get p = 0 and no say in its maximum.
//   O += P V    MFMA(srcA = V^T fragment, srcB = P fragment): P's fragment for 32
//               keys is the two 16-key accumulator tiles of S, rounded to the
//               input type and packed -- the V^T fragment is read in the same
//               key order (McTile::frag_split), so P never leaves the registers.
//               Lane l owns O[q = l % 16][d = 16 dt + 4 (l / 16) + r].
//   epilogue    O / l, rounded once to the output type.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "../../include/dmu.h"
#include "dmu_host.hpp"
#include "dmu_tiled.hpp"

namespace dmu {

struct AttnParams {
    const char *Q, *K, *V;
    char *O;
    int64_t ldq, ldk, ldv, ldo;                 // elements
    int64_t stride_q, stride_k, stride_v, stride_o;
    int32_t sq, sk, nqb;                        // query blocks per batch slice
    float scale_log2;                           // scale * log2(e)
    int64_t q_bytes, k_bytes, v_bytes;          // bytes spanned by one batch slice
    uint64_t *phases;                           // phase log (diagnostics), NULL: off
};

namespace {

constexpr int HD = 128;   // head dimension
constexpr int BQ = 256;   // query rows per workgroup
constexpr int BKEYS = 64; // keys per block

template <int T> struct Pack16;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <> struct Pack16<F16> { // two values rounded to fp16 (RNE), the first in the low half
    static __device__ __forceinline__ uint32_t two(float a, float b)
    {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
    }
};
template <> struct Pack16<BF16> {
    static __device__ __forceinline__ uint32_t two(float a, float b)
    {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    }
};

__device__ __forceinline__ float row_max4(float v) // over the lanes l, l^16, l^32, l^48
{
    // v_permlane16_swap / v_permlane32_swap with both operands v return the
    // values of lanes l and l^16 (l^32) in some order (probed): the max of the
    // pair is the max over the two lanes, without an LDS round trip
    const uint32_t x = __builtin_bit_cast(uint32_t, v);
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    const uint32_t a0 = a[0], a1 = a[1];
    v = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
    const uint32_t y = __builtin_bit_cast(uint32_t, v);
    const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
    const uint32_t b0 = b[0], b1 = b[1];
    return fmaxf(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
}

template <bool B> using Bool = std::integral_constant<bool, B>;

template <int T, int O>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_fwd(AttnParams p)
{
    typedef KcTile<BKEYS, 8, false> KT; // one 64-key x 64-value half of a K block
    typedef McTile<HD, 8> VT;           // 64 keys x 128 values of a V block
    typedef typename Out<O>::t ot;
    constexpr uint32_t KBYTES = 2 * KT::BYTES;
    constexpr uint32_t VBYTES = (VT::BYTES + 255) & ~255u;
    __shared__ __attribute__((aligned(1024))) char smem[2 * (KBYTES + VBYTES)];
    char *const kbuf = smem, *const vbuf = smem + 2 * KBYTES; // two K blocks, two V blocks

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    phase_begin(p.phases, blockIdx.x, (uint32_t)((p.sk + BKEYS - 1) / BKEYS));
    // Workgroup i runs on XCD i mod 8: renumber so that each XCD receives a
    // contiguous range, i.e. the query blocks of one batch slice share that
    // XCD's L2 for K and V.
    const uint32_t n_wg = gridDim.x, xcd = blockIdx.x % 8u, per = n_wg / 8u, extra = n_wg % 8u;
    const uint32_t wg = xcd * per + min(xcd, extra) + blockIdx.x / 8u;
    const int64_t b = wg / (uint32_t)p.nqb, q0 = (int64_t)(wg % (uint32_t)p.nqb) * BQ + wave * 32;
    const char *Qb = p.Q + b * p.stride_q * 2, *Kb = p.K + b * p.stride_k * 2, *Vb = p.V + b * p.stride_v * 2;

    // Q fragments of this wavefront's two row tiles, straight from memory
    // (rows past seq_q lie past the slice end and read as zeros).
    u32x4 qf[2][4];
    {
        const int64_t start = q0 * p.ldq * 2;
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(Qb + start, start < p.q_bytes ? (uint32_t)(p.q_bytes - start) : 0u);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qf[rt][ks] = load16s(rq, (uint32_t)((16 * rt + (lane & 15u)) * p.ldq * 2) + 64 * ks + 16 * (lane >> 4),
                                     0);
    }
    // scale * log2(e); a negative scale negates Q instead (exactly), so c >= 0
    float c = p.scale_log2;
    if (c < 0.0f) {
        c = -c;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    qf[rt][ks][e] ^= 0x80008000u;
    }

    KT tk;
    VT tv;
    tk.init(p.ldk * 2, wave, lane);
    tv.init(p.ldv * 2, HD, wave, lane);
    const int nblk = (p.sk + BKEYS - 1) / BKEYS;
    u32x4 sk_[2], sv_[VT::NL]; // a K and a V block between their global loads and their LDS writes
    auto load_k = [&](int blk) {
        const int64_t s0 = (int64_t)blk * BKEYS * p.ldk * 2;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(Kb + s0, s0 < p.k_bytes ? (uint32_t)(p.k_bytes - s0) : 0u);
#pragma unroll
        for (int h = 0; h < 2; ++h)
            sk_[h] = tk.load(0, r, h, HD * 2);
    };
    auto load_v = [&](int blk) {
        const int64_t s0 = (int64_t)blk * BKEYS * p.ldv * 2;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(Vb + s0, s0 < p.v_bytes ? (uint32_t)(p.v_bytes - s0) : 0u);
#pragma unroll
        for (int i = 0; i < VT::NL; ++i)
            sv_[i] = tv.load(i, r, 0, 0);
    };
    auto store_k = [&](char *dst) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            tk.store(0, dst + h * KT::BYTES, wave, lane, sk_[h], h, HD * 2);
    };
    auto store_v = [&](char *dst) {
#pragma unroll
        for (int i = 0; i < VT::NL; ++i)
            tv.store(i, dst, wave, lane, sv_[i], 0, 0);
    };

    f32x4 o[2][HD / 16];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int dt = 0; dt < HD / 16; ++dt)
            o[rt][dt] = f32x4{};
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.0f, 0.0f};
    f32x4 sa[2][4], sb[2][4]; // the scores of two consecutive key blocks

    // S = Q K^T for the 64 keys of the K block at kt
    auto scores = [&](f32x4 (&s)[2][4], const char *kt) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                s[rt][t] = f32x4{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            u32x4 kf[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                kf[t] = KT::frag(kt + (ks >> 1) * KT::BYTES, 16 * t, ks & 1, lane);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                    s[rt][t] = Mfma<T>::step(kf[t], qf[rt][ks], s[rt][t]);
        }
    };
    // The running maxima m (c times the largest score seen, per row) only rise
    // when a block's maximum exceeds them by more than TAU (log2 units): the
    // exponents c s - m of the softmax then stay <= TAU (p <= 2^TAU, well inside
    // the 16-bit operand formats' range), the softmax itself is unchanged (any m
    // cancels between O and l), and the rescaling of O and l by 2^(m_old - m_new)
    // is a branch almost never taken after the first blocks, instead of 64
    // multiplies per block.
    constexpr float TAU = 8.0f;
    // Each lane's maximum over its own 16 scores of a row tile decides whether a
    // raise is due (the row's maximum exceeds m + TAU exactly when one of its four
    // lanes' maxima does); the maximum across the four lanes is taken only inside
    // the rare raise.
    float bmx[2]; // this lane's maximum score in each row tile of the next block to be exponentiated
    auto block_max = [&](const f32x4 (&s)[2][4], int blk, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const int key0 = blk * BKEYS + 4 * (int)(lane >> 4);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    mx = fmaxf(mx, MASKED && key0 + 16 * t + r >= p.sk ? -INFINITY : s[rt][t][r]);
            bmx[rt] = mx;
        }
    };
    // When c bmx > m + TAU in any lane of the wavefront, every row takes m =
    // max(m, c times its block maximum) and rescales its O tiles and its sum (one
    // wavefront-uniform branch, so that every lane takes part in the cross-lane
    // maximum).  (c >= 0, so c times the maximum is the maximum of c s.)
    auto raise = [&]() {
        const bool need = bmx[0] * c > m[0] + TAU || bmx[1] * c > m[1] + TAU;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const float m_new = fmaxf(m[rt], row_max4(bmx[rt]) * c);
                const float corr = __builtin_amdgcn_exp2f(m[rt] - m_new);
                m[rt] = m_new;
                l[rt] *= corr;
#pragma unroll
                for (int dt = 0; dt < HD / 16; ++dt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        o[rt][dt][r] *= corr;
            }
        }
    };
    // Block blk's P = 2^(c s - m) packed as the operand of O += P V (tiles 2kk
    // and 2kk+1 of S make P's fragment kk), and its part of the sums l.  Only the
    // last block can hold keys past seq_k: they get no weight.
    auto softmax = [&](f32x4 (&s)[2][4], u32x4 (&pf)[2][2], int blk, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const int key0 = blk * BKEYS + 4 * (int)(lane >> 4);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float sum = 0.0f;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rt][t][r], c, -m[rt]));
                    if (MASKED)
                        e = key0 + 16 * t + r < p.sk ? e : 0.0f;
                    s[rt][t][r] = e;
                    sum += e;
                }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                pf[rt][kk] = u32x4{Pack16<T>::two(s[rt][2 * kk][0], s[rt][2 * kk][1]),
                                   Pack16<T>::two(s[rt][2 * kk][2], s[rt][2 * kk][3]),
                                   Pack16<T>::two(s[rt][2 * kk + 1][0], s[rt][2 * kk + 1][1]),
                                   Pack16<T>::two(s[rt][2 * kk + 1][2], s[rt][2 * kk + 1][3])};
            l[rt] += sum; // (after the packing: the compiler then schedules the step a little better)
        }
    };
    // O += P V for the V block at vt
    auto pv = [&](const u32x4 (&pf)[2][2], const char *vt) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int dt = 0; dt < HD / 16; ++dt) {
                const u32x4 vf = VT::frag_split(vt, 16 * dt, kk, lane);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                    o[rt][dt] = Mfma<T>::step(vf, pf[rt][kk], o[rt][dt]);
            }
    };
    // One pipelined step j (j + 1 < nblk; PAR = (j + shift) mod 2).  LDS holds
    // K block j+1 (K buffer 1-PAR) and V block j (V buffer PAR); the staging registers
    // hold K block j+2 and V block j+1.  The scores of block j+1 are computed
    // while block j's softmax runs, then O += P V for block j; K block j+2
    // goes to K buffer PAR (block j's, last read in step j-1) and V block j+1
    // to V buffer 1-PAR (block j-1's), and the next two blocks are fetched.
    auto step = [&](int j, auto par) {
        constexpr int PAR = decltype(par)::value ? 1 : 0;
        f32x4 (&s_cur)[2][4] = PAR ? sb : sa;
        f32x4 (&s_nxt)[2][4] = PAR ? sa : sb;
        raise(); // block j's maximum, taken in the previous step (or the prologue)
        scores(s_nxt, kbuf + (1 - PAR) * KBYTES);
        u32x4 pf[2][2];
        softmax(s_cur, pf, j, Bool<false>());
        block_max(s_nxt, j + 1, Bool<false>()); // (the last block's is taken again, masked, in `last`)
        pv(pf, vbuf + PAR * VBYTES);
        store_k(kbuf + PAR * KBYTES);
        store_v(vbuf + (1 - PAR) * VBYTES);
        load_k(j + 3);
        load_v(j + 2);
        stage_barrier();
    };
    // the last block (scores already in s_cur, V in buffer PAR)
    auto last = [&](int j, auto par) {
        constexpr int PAR = decltype(par)::value ? 1 : 0;
        f32x4 (&s_cur)[2][4] = PAR ? sb : sa;
        block_max(s_cur, j, Bool<true>());
        raise();
        u32x4 pf[2][2];
        softmax(s_cur, pf, j, Bool<true>());
        pv(pf, vbuf + PAR * VBYTES);
    };

    // Block j's K and V live in buffers (j + shift) mod 2 and its scores in sa
    // or sb by the same parity; shift = nblk mod 2 makes the last block odd,
    // so that the loop body is a fixed pair of steps (one step is peeled off
    // the front when the number of steps, nblk - 1, is odd).
    const int shift = nblk & 1;
    // prologue: K0 and V0, the scores of block 0, K1; K2 and V1 wait in the staging registers
    load_k(0);
    load_v(0);
    store_k(kbuf + shift * KBYTES);
    store_v(vbuf + shift * VBYTES);
    load_k(1);
    load_v(1);
    stage_barrier();
    if (shift)
        scores(sb, kbuf + KBYTES);
    else
        scores(sa, kbuf);
    if (nblk > 1) // block 0's maximum for the first step (a single block is `last`'s, masked)
        block_max(shift ? sb : sa, 0, Bool<false>());
    store_k(kbuf + (1 - shift) * KBYTES);
    load_k(2);
    stage_barrier();

    int j = 0;
    if (!shift) { // nblk even (>= 2): an odd number of steps
        step(0, Bool<false>());
        j = 1;
    }
    for (; j + 1 < nblk; j += 2) {
        step(j, Bool<true>());
        step(j + 1, Bool<false>());
    }
    last(nblk - 1, Bool<true>());
    phase_mark(p.phases, blockIdx.x, PH_LOOP);
    phase_mark(p.phases, blockIdx.x, PH_FIX);

    // O / l, each row's sum added up over the four lanes that hold its parts
    char *Ob = p.O + b * p.stride_o * (int64_t)sizeof(ot);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        float tot = l[rt];
        tot += __shfl_xor(tot, 16);
        tot += __shfl_xor(tot, 32);
        const float inv = 1.0f / tot;
        const int64_t q = q0 + 16 * rt + (lane & 15u);
        if (q >= p.sq)
            continue;
        ot *row = reinterpret_cast<ot *>(Ob) + q * p.ldo;
#pragma unroll
        for (int dt = 0; dt < HD / 16; ++dt) {
            typedef ot ov4 __attribute__((ext_vector_type(4)));
            ov4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v[r] = Out<O>::from_acc(o[rt][dt][r] * inv);
            *reinterpret_cast<ov4 *>(row + 16 * dt + 4 * (lane >> 4)) = v;
        }
    }
    phase_end(p.phases, blockIdx.x);
}

int elem_size(int t) { return t == DMU_F32 ? 4 : 2; }

int attn_validate(const dmu_attention_args *a, AttnParams *p, bool *launch)
{
    *launch = false;
    if (!a) {
        set_error("args is NULL");
        return DMU_ERR_INVALID_ARG;
    }
    if (a->batch < 0 || a->seq_q < 0 || a->seq_k < 0 || a->head_dim < 0) {
        set_error("negative size");
        return DMU_ERR_INVALID_ARG;
    }
    if (a->batch >= ((int64_t)1 << 31) || a->seq_q >= ((int64_t)1 << 31) || a->seq_k >= ((int64_t)1 << 31)) {
        set_error("size of 2^31 or more is not supported");
        return DMU_ERR_UNSUPPORTED;
    }
    if (a->head_dim != HD) {
        set_error("head_dim %lld is not supported (128 is)", (long long)a->head_dim);
        return DMU_ERR_UNSUPPORTED;
    }
    if ((a->in_type != DMU_F16 && a->in_type != DMU_BF16) ||
        (a->out_type != DMU_F32 && a->out_type != DMU_F16 && a->out_type != DMU_BF16)) {
        set_error("unsupported types (in %d, out %d)", a->in_type, a->out_type);
        return DMU_ERR_UNSUPPORTED;
    }
    if (a->batch == 0 || a->seq_q == 0)
        return DMU_OK;
    if (a->seq_k == 0) {
        set_error("seq_k == 0: the softmax of an empty row is undefined");
        return DMU_ERR_INVALID_ARG;
    }
    if (!a->Q || !a->K || !a->V || !a->O) {
        set_error("NULL operand pointer");
        return DMU_ERR_INVALID_ARG;
    }
    if (a->ldq < HD || a->ldk < HD || a->ldv < HD || a->ldo < HD) {
        set_error("leading dimension below head_dim");
        return DMU_ERR_INVALID_ARG;
    }
    if (a->stride_q < 0 || a->stride_k < 0 || a->stride_v < 0 || a->stride_o < 0) {
        set_error("negative batch stride");
        return DMU_ERR_INVALID_ARG;
    }
    const int osz = elem_size(a->out_type);
    const int64_t ext_q = (a->seq_q - 1) * a->ldq + HD, ext_k = (a->seq_k - 1) * a->ldk + HD;
    const int64_t ext_o = (a->seq_q - 1) * a->ldo + HD;
    if (a->batch > 1 && a->stride_o < ext_o) {
        set_error("stride_o lets batch slices of O overlap");
        return DMU_ERR_INVALID_ARG;
    }
    auto aligned = [](const void *ptr, int64_t ld, int64_t stride, int esz) {
        return ((uintptr_t)ptr % 16) == 0 && (ld * esz) % 16 == 0 && (stride * esz) % 16 == 0;
    };
    const bool b1 = a->batch > 1;
    if (!aligned(a->Q, a->ldq, b1 ? a->stride_q : 0, 2) || !aligned(a->K, a->ldk, b1 ? a->stride_k : 0, 2) ||
        !aligned(a->V, a->ldv, b1 ? a->stride_v : 0, 2) || !aligned(a->O, a->ldo, b1 ? a->stride_o : 0, osz)) {
        set_error("operands must have 16-byte aligned pointers, rows and batch strides");
        return DMU_ERR_UNSUPPORTED;
    }
    const int64_t slice_max = ((int64_t)1 << 31);
    if (ext_q * 2 >= slice_max || ext_k * 2 >= slice_max || ((a->seq_k - 1) * a->ldv + HD) * 2 >= slice_max) {
        set_error("a batch slice of 2 GiB or more is not supported");
        return DMU_ERR_UNSUPPORTED;
    }
    // O may not overlap the inputs
    auto span = [&](const void *ptr, int64_t stride, int64_t ext, int esz, uintptr_t *lo, uintptr_t *hi) {
        *lo = (uintptr_t)ptr;
        *hi = *lo + (uintptr_t)(((a->batch - 1) * (b1 ? stride : 0) + ext) * esz);
    };
    uintptr_t o0, o1, x0, x1;
    span(a->O, a->stride_o, ext_o, osz, &o0, &o1);
    const struct { const void *p; int64_t stride, ext; } ins[3] = {
        {a->Q, a->stride_q, ext_q}, {a->K, a->stride_k, ext_k}, {a->V, a->stride_v, (a->seq_k - 1) * a->ldv + HD}};
    for (const auto &x : ins) {
        span(x.p, x.stride, x.ext, 2, &x0, &x1);
        if (o0 < x1 && x0 < o1) {
            set_error("O overlaps an input");
            return DMU_ERR_INVALID_ARG;
        }
    }
    const int64_t nqb = (a->seq_q + BQ - 1) / BQ;
    if (nqb * a->batch >= ((int64_t)1 << 31)) {
        set_error("too many workgroups for one launch");
        return DMU_ERR_UNSUPPORTED;
    }
    p->Q = static_cast<const char *>(a->Q);
    p->K = static_cast<const char *>(a->K);
    p->V = static_cast<const char *>(a->V);
    p->O = static_cast<char *>(a->O);
    p->ldq = a->ldq;
    p->ldk = a->ldk;
    p->ldv = a->ldv;
    p->ldo = a->ldo;
    p->stride_q = b1 ? a->stride_q : 0;
    p->stride_k = b1 ? a->stride_k : 0;
    p->stride_v = b1 ? a->stride_v : 0;
    p->stride_o = b1 ? a->stride_o : 0;
    p->sq = (int32_t)a->seq_q;
    p->sk = (int32_t)a->seq_k;
    p->nqb = (int32_t)nqb;
    p->scale_log2 = a->scale * 1.4426950408889634f;
    p->q_bytes = ext_q * 2;
    p->k_bytes = ext_k * 2;
    p->v_bytes = ((a->seq_k - 1) * a->ldv + HD) * 2;
    *launch = true;
    return DMU_OK;
}

template <int T, int O> hipError_t go(const AttnParams &p, int64_t grid, hipStream_t s)
{
    hipLaunchKernelGGL((attn_fwd<T, O>), dim3((uint32_t)grid), dim3(512), 0, s, p);
    return hipGetLastError();
}

} // namespace
} // namespace dmu

using namespace dmu;

extern "C" int dmu_attention_check(const dmu_attention_args *args)
{
    clear_error();
    AttnParams p{};
    bool launch;
    return attn_validate(args, &p, &launch);
}

extern "C" int dmu_attention(const dmu_attention_args *args, void *stream)
{
    clear_error();
    AttnParams p{};
    bool launch;
    int rc = attn_validate(args, &p, &launch);
    if (rc != DMU_OK || !launch)
        return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int64_t grid = (int64_t)p.nqb * args->batch;
    if ((rc = phase_reserve((size_t)grid, 4, "dmu_attention", &p.phases)) != DMU_OK)
        return rc;
    hipError_t e;
    const bool bf = args->in_type == DMU_BF16;
    switch (args->out_type) {
    case DMU_F32: e = bf ? go<BF16, F32>(p, grid, s) : go<F16, F32>(p, grid, s); break;
    case DMU_F16: e = bf ? go<BF16, F16>(p, grid, s) : go<F16, F16>(p, grid, s); break;
    default: e = bf ? go<BF16, BF16>(p, grid, s) : go<F16, BF16>(p, grid, s); break;
    }
    if (e != hipSuccess) {
        set_error("dmu_attention: launch failed: %s", hipGetErrorString(e));
        return DMU_ERR_HIP;
    }
    return DMU_OK;
}
