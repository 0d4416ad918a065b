// Output epilogues shared by the projection passes (ee_proj.hip: rows staged
// 8 at a time; ee_wide.hip: up to 64 rows on matrix cores).
#pragma once
#include "ee_internal.h"
#include "ee_device.h"

namespace ee {

// QKV epilogue for row n of sequence seq at position pos: v is this row's
// value, u its RoPE partner's (row n -/+ hd/2).  q and k are rounded to bf16,
// rotated in float32 and rounded again; k and v go to the shared cache slot of
// the position.  The epilogue's inputs from memory (the rotation factors of
// the row's element and the slot's occupancy count) are requested by qkv_pre,
// which a pass calls when the row is known, long before the row's value is.
struct QkvPre {
  float c, s;  // cos and sin of the row's element at pos (q and k rows)
  int occ;     // occupancy count of the slot (read by the row that updates it)
};

__device__ __forceinline__ QkvPre qkv_pre(const ProjArgs& a, int seq, int n, int pos) {
  const int hd = a.hd, half = hd >> 1;
  const int head = n >> a.hd_log2;
  const int e = n & (hd - 1);
  const int i = e < half ? e : e - half;  // in bounds for every row (v rows do not use it)
  QkvPre r;
  r.c = a.cosT[(size_t)pos * half + i];
  r.s = a.sinT[(size_t)pos * half + i];
  r.occ = 0;
  if (a.occ_l && head == a.H && e == 0) r.occ = a.occ_l[(size_t)seq * a.S + pos];
  return r;
}

__device__ __forceinline__ void qkv_out(const ProjArgs& a, int seq, int n, float v, float u, int pos,
                                        const QkvPre& pre) {
  const int hd = a.hd, half = hd >> 1;
  const int head = n >> a.hd_log2;
  const int e = n & (hd - 1);
  if (head < a.H + a.Hkv) {
    const float x = bf2f(f2bf(v)), y = bf2f(f2bf(u));
    const float r = e < half ? x * pre.c - y * pre.s : x * pre.c + y * pre.s;  // (x1 c - x2 s, x2 c + x1 s)
    const uint16_t o = (uint16_t)f2bf(r);
    if (head < a.H) {
      a.qrot[((size_t)seq * a.H + head) * hd + e] = o;
    } else {
      const int kh = head - a.H;
      a.Kl[(((size_t)seq * a.Hkv + kh) * a.S + pos) * hd + e] = o;
      if (a.occ_l && kh == 0 && e == 0) a.occ_l[(size_t)seq * a.S + pos] = pre.occ + 1;
    }
  } else {
    const int vh = head - a.H - a.Hkv;
    a.Vl[(((size_t)seq * a.Hkv + vh) * a.S + pos) * hd + e] = (uint16_t)f2bf(v);
  }
}

__device__ __forceinline__ void qkv_out(const ProjArgs& a, int seq, int n, float v, float u) {
  const int pos = a.lens[seq];
  qkv_out(a, seq, n, v, u, pos, qkv_pre(a, seq, n, pos));
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace ee
