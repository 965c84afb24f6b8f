// The hyper-connection split (readings of dispatch_hc_split_sinkhorn on the
// hf2q ffn_forward.rs page, stated in moe_ffn.h): a row's mix sums and sum
// of squares -> pre = sigmoid, post = 2 * sigmoid, comb = Sinkhorn rounds
// of exp.  Used by the wrapper's pre launch (more than 4 rows) and by the
// decode head, which splits a 1-4-row call's mixes itself.
#pragma once

#include "device.h"

namespace moe {

// Up to 4 rows by one whole wave (every lane active for the DPP moves):
// lane 16 * rr + 4j + i holds comb entry (j, i) of row rr through the
// Sinkhorn rounds (row sums over the lanes of one j: a quad; column sums
// over the lanes of one i: 4 apart, reached by rotating the 16-lane row by
// 4 and by 8; each division a reciprocal and a multiply, within 2 ulp).
// sums + rr * spitch: row rr's (2 + HC) * HC mix sums, then its sum of
// squares over `count` inputs.  Writes the maps of rows rr < nrr to maps +
// rr * mpitch and, when `mixes` is not null, the normalised mixes to
// mixes + rr * (2 + HC) * HC.
template <int HC>
__device__ __forceinline__ void hc_split_rows(const float* sums, int spitch, int nrr, float count, float eps,
                                              const float* scale, const float* base, int iters, float* maps,
                                              int mpitch, float* mixes) {
  constexpr int MW = (2 + HC) * HC;
  const int lane = threadIdx.x % kWave, rr = lane / 16, j = (lane / 4) % 4, i = lane % 4;
  const bool row_ok = rr < nrr;
  const float* sr = sums + (row_ok ? rr : 0) * spitch;  // every lane reads a valid row
  const float rinv = 1.0f / sqrtf(sr[MW] / count + eps);
  const bool in = row_ok && j < HC && i < HC;
  float* mr = maps + rr * mpitch;
  if (in && i == 0) {  // pre_j and post_j
    mr[j] = 1.0f / (1.0f + expf(-(scale[0] * (sr[j] * rinv) + base[j])));
    mr[HC + j] = 2.0f / (1.0f + expf(-(scale[1] * (sr[HC + j] * rinv) + base[HC + j])));
  }
  float c = 0.f;
  if (in) c = expf(scale[2] * (sr[2 * HC + j * HC + i] * rinv) + base[2 * HC + j * HC + i]);
  for (int it = 0; it < iters; ++it) {
    float rsum = c + dpp_f32<0xB1>(c);
    rsum += dpp_f32<0x4E>(rsum);
    c = in ? c * __builtin_amdgcn_rcpf(rsum) : 0.f;
    float csum = c + dpp_f32<0x124>(c);
    csum += dpp_f32<0x128>(csum);
    c = in ? c * __builtin_amdgcn_rcpf(csum) : 0.f;
  }
  if (in) mr[2 * HC + j * HC + i] = c;
  if (mixes && row_ok)
    for (int m = lane % 16; m < MW; m += 16) mixes[rr * MW + m] = sr[m] * rinv;
}

// The same for a run-time stream count (1..4).
__device__ __forceinline__ void hc_split_rows_n(int hc, const float* sums, int spitch, int nrr, float count,
                                                float eps, const float* scale, const float* base, int iters,
                                                float* maps, int mpitch, float* mixes) {
  switch (hc) {
    case 1: hc_split_rows<1>(sums, spitch, nrr, count, eps, scale, base, iters, maps, mpitch, mixes); break;
    case 2: hc_split_rows<2>(sums, spitch, nrr, count, eps, scale, base, iters, maps, mpitch, mixes); break;
    case 3: hc_split_rows<3>(sums, spitch, nrr, count, eps, scale, base, iters, maps, mpitch, mixes); break;
    default: hc_split_rows<4>(sums, spitch, nrr, count, eps, scale, base, iters, maps, mpitch, mixes); break;
  }
}

}  // namespace moe
