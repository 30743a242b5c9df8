/* Calls every entry point of libss2d.so (host code built with AddressSanitizer
 * and UndefinedBehaviorSanitizer) with arguments that validation rejects, and
 * with valid arguments on a machine without a GPU (SS2D_ERR_NO_DEVICE), and
 * runs ss2d_describe over many shapes.  Fake addresses are never dereferenced.
 * Prints one line per check and exits nonzero on the first unexpected code. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ss2d.h"

static int failures = 0;
static void expect(const char* what, int got, int want) {
  printf("%-48s %3d (want %3d)\n", what, got, want);
  if (got != want) ++failures;
}

int main(void) {
  const uintptr_t base = (uintptr_t)1 << 40;
  void* p[24];
  for (int i = 0; i < 24; ++i) p[i] = (void*)(base + (uintptr_t)i * ((uintptr_t)1 << 34));
  const float* fp[24];
  for (int i = 0; i < 24; ++i) fp[i] = (const float*)p[i];

  /* forward and its siblings */
  expect("forward valid", ss2d_forward(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[7], 2, 3, 4, 5, 16, 0, 0), -7);
  expect("forward null x", ss2d_forward(0, p[1], fp[2], fp[3], p[4], p[5], fp[6], p[7], 2, 3, 4, 5, 16, 0, 0), -1);
  expect("forward H = 0", ss2d_forward(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[7], 2, 3, 0, 5, 16, 0, 0), -2);
  expect("forward huge", ss2d_forward(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[7], (int64_t)1 << 40, 1 << 20,
                                      8, 8, 16, 0, 0), -2);
  expect("forward N = 257", ss2d_forward(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[7], 2, 3, 4, 5, 257, 0, 0), -3);
  expect("forward dtype 7", ss2d_forward(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[7], 2, 3, 4, 5, 16, 7, 0), -4);
  expect("forward alias", ss2d_forward(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[0], 2, 3, 4, 5, 16, 0, 0), -5);
  expect("forward misaligned", ss2d_forward((char*)p[0] + 2, p[1], fp[2], fp[3], p[4], p[5], fp[6], p[7], 2, 3, 4, 5,
                                            16, 0, 0), -6);
  expect("forward offset base (scalar path)", ss2d_forward((char*)p[0] + 4, p[1], fp[2], fp[3], p[4], p[5], fp[6],
                                                           p[7], 2, 3, 4, 4, 256, 0, 0), -7);
  expect("forward_lanes bad", ss2d_forward_lanes(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[7], 2, 3, 4, 5, 16, 0,
                                                 48, 0), -2);
  expect("forward_lanes 64", ss2d_forward_lanes(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[7], 2, 3, 4, 5, 16, 0,
                                                64, 0), -7);
  expect("forward_noalloc over the limit", ss2d_forward_noalloc(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[7], 64,
                                                                384, 28, 28, 16, 1, 0), -9);
  expect("forward_noalloc valid", ss2d_forward_noalloc(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[7], 2, 3, 4, 5,
                                                       16, 0, 0), -7);
  expect("bidir valid", ss2d_bidir_forward(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[7], 2, 3, 20, 16, 1, 0), -7);
  expect("bidir L = 0", ss2d_bidir_forward(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[7], 2, 3, 0, 16, 0, 0), -2);

  /* projections, epilogue, backward */
  expect("project valid", ss2d_project(p[0], fp[8], fp[9], p[1], p[4], p[5], 2, 3, 4, 5, 16, 2, 0, 0), -7);
  expect("project rank 0", ss2d_project(p[0], fp[8], fp[9], p[1], p[4], p[5], 2, 3, 4, 5, 16, 0, 0, 0), -2);
  expect("from_x valid", ss2d_forward_from_x(p[0], fp[8], fp[9], fp[2], fp[3], fp[6], p[7], 2, 3, 4, 5, 16, 2, 0, 0),
         -7);
  expect("channel_last valid", ss2d_channel_last(p[0], fp[10], fp[11], 1e-5f, 1, p[12], 2, 3, 4, 5, 0, 0), -7);
  expect("channel_last bad eps", ss2d_channel_last(p[0], fp[10], fp[11], -1.f, 1, p[12], 2, 3, 4, 5, 0, 0), -2);
  expect("backward valid", ss2d_backward(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[13], p[14], p[15],
                                         (float*)p[16], (float*)p[17], p[18], p[19], (float*)p[20], 2, 3, 4, 5, 16, 0, 0),
         -7);
  expect("backward N = 257", ss2d_backward(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[13], p[14], p[15],
                                           (float*)p[16], (float*)p[17], p[18], p[19], (float*)p[20], 2, 3, 4, 5, 257, 0,
                                           0), -3);
  expect("backward N = 17", ss2d_backward(p[0], p[1], fp[2], fp[3], p[4], p[5], fp[6], p[13], p[14], p[15],
                                          (float*)p[16], (float*)p[17], p[18], p[19], (float*)p[20], 2, 3, 4, 5, 17, 0,
                                          0), -7);
  ss2d_peaks pk;
  expect("measure_peaks bad size", ss2d_measure_peaks(&pk, 1000, 0), -2);

  /* plans and strings */
  char buf[512];
  const int64_t shapes[][6] = {{1, 16, 8, 8, 16, 0},      {32, 192, 56, 56, 16, 0}, {32, 768, 14, 14, 16, 0},
                               {64, 384, 28, 28, 16, 1},  {2, 192, 256, 256, 16, 0}, {1, 11, 96, 100, 16, 0},
                               {1, 1, 1, 1, 1, 0},        {3, 17, 33, 31, 256, 1},  {2, 5, 1, 40000, 20, 1}};
  for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
    const int64_t* s = shapes[i];
    const int rc = ss2d_describe(s[0], s[1], s[2], s[3], s[4], (int)s[5], buf, sizeof buf);
    expect("describe", rc, 0);
    if (strlen(buf) == 0) ++failures;
    for (int lanes = 16; lanes <= 64; lanes *= 2)
      expect("describe_lanes", ss2d_describe_lanes(s[0], s[1], s[2], s[3], s[4], (int)s[5], lanes, buf, sizeof buf), 0);
  }
  expect("describe tiny buffer", ss2d_describe(2, 3, 4, 5, 16, 0, buf, 1), 0);
  for (int c = 1; c >= -10; --c)
    if (ss2d_status_string(c) == 0) ++failures;
  if (ss2d_last_hip_error() == 0) ++failures;
  printf("failures: %d\n", failures);
  return failures ? 1 : 0;
}
