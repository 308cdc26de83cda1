"""CSA2 CPU oracle package. Test infrastructure only; the product never imports it."""
