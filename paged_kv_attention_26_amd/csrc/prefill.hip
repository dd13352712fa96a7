// Chunked-prefill attention (MFMA) -- not built yet.
#include "pa_internal.h"
