// Batched W2 phase on the matrix cores (bf16 W2, r = 32 * KS), for the
// stepwise launches at B > 8: per position p,
//   L_p[b][v] = L_base[b][p][v] + sum_k W2[v][k] u_p[b][k],  t_p[b] = argmax_v L_p[b][v]
// (paper.oopus.info review, section 二, 第二步 Domino Head: low-rank logit
// correction added to the base logits; news.sig.ai article, section
// "Domino怎么做": greedy decoding).  Built for 256-thread blocks.
#define DH_NT 256
#define DH_NS dh256
#include "dh_phases.h"
#include "dh_batched.h"

namespace DH_NS {

// Work split.  A block takes a batch tile of up to 128 rows (bt) and a
// contiguous vocabulary range (vb of nvb); its four waves take 32-row batch
// groups of the tile and split the range into 64-row chunks when the tile has
// fewer than four groups.  A wave keeps its 32 batch rows of u in registers
// as four matrix-core A operands: A tile a holds batch rows a*8 .. a*8+7 as
// bf16 hi parts in rows 0..7 and lo parts (u - hi) in rows 8..15, so the two
// results of a batch row come out 32 lanes apart and are added (the same
// operand form and order as the resident kernel, so both give the same
// values).  For each 64-row chunk the wave multiplies the A tiles with four
// 16-row W2 tiles (v_mfma_f32_16x16x32_bf16, D = A W2_tile^T), adds hi + lo,
// packs two A tiles per register and folds L_base, the optional L_final
// store and the greedy argmax.  Each lane keeps the running best of its eight
// batch rows; at the end the 16 lanes of a batch row reduce it and one lane
// folds it into the partial key slot of group blockIdx % NG with an atomic max.
template <int KS>
__global__ __launch_bounds__(NT) void k_w2_mfma(Params p, int pos)
{
    const int r = 32 * KS;
    const int B = p.B, V = p.V;
    const int nbt = (B + 127) / 128;
    const int bt = blockIdx.x % nbt, vb = blockIdx.x / nbt, nvb = gridDim.x / nbt;
    if (vb >= nvb)
        return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rows = B - bt * 128 < 128 ? B - bt * 128 : 128;  // batch rows of this tile
    const int ng = rows <= 32 ? 1 : rows <= 64 ? 2 : 4;         // 32-row groups (waves per chunk)
    const int grp = wave % ng, vs = wave / ng, nvs = 4 / ng;
    const int row0 = bt * 128 + grp * 32;                       // first batch row of the wave
    const long long v0 = static_cast<long long>(V) * vb / nvb;
    const int n = static_cast<int>(static_cast<long long>(V) * (vb + 1) / nvb - v0);
    const int col = lane & 15;
    const int g = blockIdx.x % NG;

    // A operands: u of batch row row0 + a*8 + (col & 7), hi part for col < 8, lo part otherwise
    uint4 ua[4][KS];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int b = row0 + a * 8 + (col & 7);
        const bool hi = col < 8;
        const float *src = p.u_buf + static_cast<size_t>(b < B ? b : 0) * r + (lane >> 4) * 8;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            float x[8];
            if (b < B) {
                const float4 x0 = *reinterpret_cast<const float4 *>(src + kk * 32);
                const float4 x1 = *reinterpret_cast<const float4 *>(src + kk * 32 + 4);
                x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
                x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    x[j] = 0.f;
            }
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t xh = bf16_rne_bits(x[j]);
                h[j] = hi ? xh : bf16_rne_bits(x[j] - __uint_as_float(xh << 16));
            }
            ua[a][kk] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
        }
    }

    // lane's batch rows in the packed epilogue: pair pp packs A tiles 2pp (lanes 0..31)
    // and 2pp+1 (lanes 32..63); row i of four per lane
    int brow[2][4];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            brow[pp][i] = row0 + (2 * pp + (lane >> 5)) * 8 + ((lane >> 4) & 1) * 4 + i;
    LaneBest best[2][4];

#pragma unroll 1
    for (int c0 = vs * 64; c0 < n; c0 += nvs * 64) {
        // L_base of the epilogue values, issued first
        float lb[2][4][4];  // [pp][vt][i]
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int vt = 0; vt < 4; ++vt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int b = brow[pp][i], vr = c0 + vt * 16 + col;
                    const size_t o = (static_cast<size_t>(b < B ? b : 0) * p.K + pos) * V + v0 + (vr < n ? vr : 0);
                    lb[pp][vt][i] = p.L_base[o];
                }
        f32x4_t acc[4][4];  // [a][vt]
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int vt = 0; vt < 4; ++vt)
                acc[a][vt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            uint4 wb[4];
#pragma unroll
            for (int vt = 0; vt < 4; ++vt) {
                const int vr = c0 + vt * 16 + col;
                wb[vt] = vr < n ? ld16<bf16s>(p.W2, static_cast<size_t>(v0 + vr) * r + kk * 32 + (lane >> 4) * 8)
                                : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int vt = 0; vt < 4; ++vt)
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    acc[a][vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ua[a][kk]),
                                                                        __builtin_bit_cast(bf16x8_t, wb[vt]),
                                                                        acc[a][vt], 0, 0, 0);
        }
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int vt = 0; vt < 4; ++vt) {
                const int vr = c0 + vt * 16 + col;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x0 = w2_hilo(acc[2 * pp][vt], i), x1 = w2_hilo(acc[2 * pp + 1][vt], i);
                    const auto d = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x1), false,
                                                                    false);
                    const int b = brow[pp][i];
                    const bool ok = b < B && vr < n;
                    float *lf = p.L_final ? p.L_final + (static_cast<size_t>(b) * p.K + pos) * V + v0 : nullptr;
                    w2_key(__uint_as_float(d[0]), lb[pp][vt][i], lf, static_cast<int>(v0), vr, ok, best[pp][i]);
                }
            }
    }
    // each batch row's best over its 16 lanes, folded into the partial key slot
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint64_t key = best[pp][i].ord ? (static_cast<uint64_t>(best[pp][i].ord) << 32) |
                                                 (0xFFFFFFFFu - best[pp][i].idx)
                                           : 0ull;
            key = max_u64(key, dpp_u64<DPP_QUAD_XOR1>(key));
            key = max_u64(key, dpp_u64<DPP_QUAD_XOR2>(key));
            key = max_u64(key, dpp_u64<DPP_HALF_MIRROR>(key));
            key = max_u64(key, dpp_u64<DPP_ROW_MIRROR>(key));
            const int b = brow[pp][i];
            if (col == 0 && b < B && key)
                __hip_atomic_fetch_max(key_slot(p, pos, g, b), key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
}

constexpr int BAT_KS = 8;  // r = 256

}  // namespace DH_NS

namespace dhbat {

using namespace dh256;

int r_supported() { return 32 * BAT_KS; }
int threads() { return NT; }
const void *w2_kernel() { return reinterpret_cast<const void *>(&k_w2_mfma<BAT_KS>); }
// one block per compute unit: batch tiles times vocabulary ranges
int w2_grid(int B, int cus)
{
    const int nbt = (B + 127) / 128;
    const int nvb = (cus + nbt - 1) / nbt;
    return nbt * nvb;
}

}  // namespace dhbat
