// Shared-prefix tail-prefill attention: the second build of the kernel in blink_attention.hip,
// compiled with the compiler's default instruction scheduler, for prefix-free requests of short
// tails (the main build's scheduler favours the matrix-bound launches). It holds the kernel and
// blink_attention_plain_launch only; the library's entry points live in the main build.
#define BLINK_ATTENTION_PLAIN 1
#include "blink_attention.hip"
