// BOS-aligned best-fit packing of a document stream into fixed-length rows
// (host code; the loader step that produces the token rows a training step
// consumes).
//
// [CT50] "4. Carregamento de Dados": every row starts with BOS, rows are
// filled with whole documents chosen best-fit, and when no buffered document
// fits one is cut to fill the row. Here: before each choice the buffer is
// topped up from the stream to its capacity; the longest buffered document
// that fits the space left is placed whole (the earliest among equal
// lengths); if none fits, the shortest (earliest among equals) is cut to the
// space left, its tail dropped. A chosen document leaves the buffer and the
// others keep their arrival order. Documents carry their own leading BOS, so
// a row starts with BOS because it starts with a document's first token.
#include <stdint.h>
#include <string.h>

#include "../../include/gpt.h"

extern "C" gpt_status gpt_pack_best_fit(const int32_t* tokens, const int64_t* offsets, int64_t n_docs,
                                        int64_t* buffer, int32_t* buffer_count, int32_t buffer_cap,
                                        int64_t* next_doc, int32_t rows, int32_t row_len, int32_t* out,
                                        int64_t* tokens_cut) {
  if (!tokens || !offsets || !buffer || !buffer_count || !next_doc || !out) return GPT_EINVAL;
  if (n_docs < 0 || buffer_cap < 1 || rows < 0 || row_len < 1) return GPT_EINVAL;
  int32_t count = *buffer_count;
  int64_t next = *next_doc;
  if (count < 0 || count > buffer_cap || next < 0 || next > n_docs) return GPT_EINVAL;
  for (int32_t i = 0; i < count; ++i)
    if (buffer[i] < 0 || buffer[i] >= n_docs || offsets[buffer[i] + 1] <= offsets[buffer[i]]) return GPT_EINVAL;
  auto length = [&](int64_t d) { return offsets[d + 1] - offsets[d]; };
  int64_t cut = 0;
  gpt_status st = GPT_OK;
  for (int32_t r = 0; r < rows && st == GPT_OK; ++r) {
    int32_t* row = out + (int64_t)r * row_len;
    int64_t remaining = row_len;
    while (remaining > 0) {
      while (count < buffer_cap && next < n_docs && offsets[next + 1] > offsets[next]) buffer[count++] = next++;
      if (count < buffer_cap && next < n_docs) {
        st = GPT_EDATA;  // an empty document, or offsets that decrease
        break;
      }
      if (count == 0) {
        st = GPT_EDATA;  // the stream ran out in mid-row
        break;
      }
      int32_t pick = -1;
      int64_t pick_len = 0;
      for (int32_t i = 0; i < count; ++i) {
        const int64_t n = length(buffer[i]);
        if (n <= remaining && n > pick_len) {
          pick = i;
          pick_len = n;
        }
      }
      int64_t take;
      if (pick >= 0) {
        take = pick_len;
      } else {
        pick = 0;
        for (int32_t i = 1; i < count; ++i)
          if (length(buffer[i]) < length(buffer[pick])) pick = i;
        take = remaining;
        cut += length(buffer[pick]) - take;
      }
      const int64_t d = buffer[pick];
      memcpy(row + (row_len - remaining), tokens + offsets[d], (size_t)take * sizeof(int32_t));
      memmove(buffer + pick, buffer + pick + 1, (size_t)(count - pick - 1) * sizeof(int64_t));
      --count;
      remaining -= take;
    }
  }
  // The state is written back on error too, so it stays consistent with the
  // buffer contents (rows up to the failing one are complete).
  *buffer_count = count;
  *next_doc = next;
  if (tokens_cut) *tokens_cut = cut;
  return st;
}
